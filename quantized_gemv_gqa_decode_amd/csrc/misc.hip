// misc.hip -- the small kernels of the decode step and the weight quantizers.
#include <math.h>

#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

// ---------------------------------------------------------------- RMSNorm --
// GroupedRMSNorm ([k2-burn] "Model shape": layernorm_num_groups): one block per
// (row, group); y = x / sqrt(mean(x^2) + eps) * gamma.  Groups of up to
// RMS_V * 1024 elements (float4-aligned) are held in registers: every load of
// the group and of gamma is issued before the first is used, so the kernel
// pays one memory round trip instead of one per loop step; other groups take
// the strided loop.
constexpr int RMS_V = 8;                        // float4s per thread held in registers

__device__ __forceinline__ bool rms_vec_ok(int gs, const float *xr, const float *gm)
{
    return gs % 4 == 0 && gs <= RMS_V * 4 * K2_BLOCK && ((uintptr_t)xr & 15u) == 0 && ((uintptr_t)gm & 15u) == 0;
}

// the block's sum of x^2 over its group -> 1 / rms (every thread)
__device__ __forceinline__ float rms_scale(float ss, int gs, float eps)
{
    __shared__ float red[K2_WAVES_PER_BLOCK];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < K2_WAVES_PER_BLOCK; ++w) t += red[w];
    return 1.0f / sqrtf(t / (float)gs + eps);
}

// y (or its bf16 hi / lo planes) for the block's group; OUT(i, value) stores
// element i of the group
template <class Out>
__device__ __forceinline__ void rms_group(const float *xr, const float *gm, int gs, float eps, Out out)
{
    if (rms_vec_ok(gs, xr, gm)) {
        const int n4 = gs / 4;
        float4 xv[RMS_V], gv[RMS_V];
#pragma unroll
        for (int v = 0; v < RMS_V; ++v) {
            const int i = v * K2_BLOCK + threadIdx.x;
            const int ii = i < n4 ? i : 0;
            xv[v] = reinterpret_cast<const float4 *>(xr)[ii];
            gv[v] = reinterpret_cast<const float4 *>(gm)[ii];
        }
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < RMS_V; ++v)
            if (v * K2_BLOCK + (int)threadIdx.x < n4)
                ss += xv[v].x * xv[v].x + xv[v].y * xv[v].y + xv[v].z * xv[v].z + xv[v].w * xv[v].w;
        const float r = rms_scale(ss, gs, eps);
#pragma unroll
        for (int v = 0; v < RMS_V; ++v) {
            const int i = v * K2_BLOCK + threadIdx.x;
            if (i < n4) {
                out(4 * i, xv[v].x * r * gv[v].x);
                out(4 * i + 1, xv[v].y * r * gv[v].y);
                out(4 * i + 2, xv[v].z * r * gv[v].z);
                out(4 * i + 3, xv[v].w * r * gv[v].w);
            }
        }
    } else {
        float ss = 0.f;
        for (int i = threadIdx.x; i < gs; i += K2_BLOCK) ss += xr[i] * xr[i];
        const float r = rms_scale(ss, gs, eps);
        for (int i = threadIdx.x; i < gs; i += K2_BLOCK) out(i, xr[i] * r * gm[i]);
    }
}

__global__ __launch_bounds__(K2_BLOCK) void rmsnorm_grouped_kernel(const float *x, const float *gamma,
                                                                   float *y, int hidden, int groups,
                                                                   float eps)
{
    const int row = blockIdx.x / groups, g = blockIdx.x % groups, gs = hidden / groups;
    const int64_t o = (int64_t)row * hidden + (int64_t)g * gs;
    float *yr = y + o;
    rms_group(x + o, gamma + (int64_t)g * gs, gs, eps, [&](int i, float v) { yr[i] = v; });
}

// The same rows written as bf16 hi / lo planes (hi = bf16(y), lo = bf16(y -
// hi)), the form the matrix-core products of a prefill chunk read.
__global__ __launch_bounds__(K2_BLOCK) void rmsnorm_planes_kernel(const float *x, const float *gamma,
                                                                  uint16_t *yh, uint16_t *yl, int hidden,
                                                                  int groups, float eps)
{
    const int row = blockIdx.x / groups, g = blockIdx.x % groups, gs = hidden / groups;
    const int64_t o = (int64_t)row * hidden + (int64_t)g * gs;
    rms_group(x + o, gamma + (int64_t)g * gs, gs, eps, [&](int i, float v) {
        const uint16_t h = f32_to_bf16_rne(v);
        yh[o + i] = h;
        yl[o + i] = f32_to_bf16_rne(v - bf16_to_f32(h));
    });
}

// ------------------------------------------------------------------- RoPE --
// cos/sin of pos * theta^(-2i/hd), computed in fp64 and stored as fp32.
__global__ void rope_table_kernel(float *cs, int cap, int hd, double theta)
{
    const int half = hd / 2;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)cap * half) return;
    const int p = (int)(t / half), i = (int)(t % half);
    const double inv = pow(theta, -2.0 * (double)i / (double)hd);
    const double ang = (double)p * inv;
    cs[t * 2] = (float)cos(ang);
    cs[t * 2 + 1] = (float)sin(ang);
}

// split-half rotation of n_heads heads of size hd, in place; one thread per pair
__global__ void rope_kernel(float *q, float *k, const float *cs, int n_qh, int n_kv, int hd, int pos)
{
    const int half = hd / 2;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (n_qh + n_kv) * half) return;
    const int h = t / half, i = t % half;
    float *u = (h < n_qh) ? q + (int64_t)h * hd : k + (int64_t)(h - n_qh) * hd;
    const float c = cs[((int64_t)pos * half + i) * 2], s = cs[((int64_t)pos * half + i) * 2 + 1];
    const float a = u[i], b = u[i + half];
    u[i] = a * c - b * s;
    u[i + half] = a * s + b * c;
}

// ------------------------------------------------------------------ embed --
// h = fp32(E[token]); the token comes from the host (token >= 0) or from
// device memory (d_token).  A device token outside [0, vocab) sets *d_err and
// is replaced by 0 so that every later kernel still runs to completion.
__global__ void embed_kernel(int embdt, const void *E, int H, int vocab, int token,
                             const int32_t *d_token, int32_t *d_err, float *h)
{
    int tok = token;
    if (d_token) {
        tok = *d_token;
        if (tok < 0 || tok >= vocab) {
            if (d_err && threadIdx.x == 0 && blockIdx.x == 0) *d_err = K2_ERANGE;
            tok = 0;
        }
    }
    const int64_t base = (int64_t)tok * H;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < H; i += gridDim.x * blockDim.x)
        h[i] = embdt == K2_BF16 ? bf16_to_f32(((const uint16_t *)E)[base + i])
                                : ((const float *)E)[base + i];
}

int embed_launch(int embdt, const void *E, int H, int vocab, int token, const int32_t *d_token,
                 int32_t *d_err, float *h, hipStream_t st)
{
    int blocks = (H + K2_BLOCK - 1) / K2_BLOCK;
    if (blocks > 64) blocks = 64;
    hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(K2_BLOCK), 0, st, embdt, E, H, vocab, token,
                       d_token, d_err, h);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// ------------------------------------------------------------- quantizers --
// fp8 E4M3FN per output row ([k2-burn] "Quantization"): one block per row.
__global__ __launch_bounds__(K2_BLOCK) void quant_fp8_rows_kernel(const uint16_t *W, uint8_t *codes,
                                                                  float *scale, int K)
{
    __shared__ float red[K2_WAVES_PER_BLOCK];
    const int64_t n = blockIdx.x;
    const uint16_t *row = W + n * K;
    float m = 0.f;
    for (int k = threadIdx.x; k < K; k += K2_BLOCK) m = fmaxf(m, fabsf(bf16_to_f32(row[k])));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < K2_WAVES_PER_BLOCK; ++w) amax = fmaxf(amax, red[w]);
    const float s = amax / 448.0f;                 // IEEE fp32 division
    if (threadIdx.x == 0) scale[n] = s;
    for (int k = threadIdx.x; k < K; k += K2_BLOCK) {
        uint8_t c = 0;
        if (amax != 0.f) c = f32_to_e4m3(bf16_to_f32(row[k]) / s);
        codes[n * K + k] = c;
    }
}

// MXFP4 (OCP Microscaling: E2M1, 32-column blocks, E8M0): one thread per block.
__global__ void quant_mxfp4_kernel(const uint16_t *W, uint8_t *q, uint8_t *e8m0, int64_t n_blocks,
                                   int K)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const int64_t nb_row = K / 32;
    const int64_t n = b / nb_row, bb = b % nb_row;
    const uint16_t *src = W + n * K + bb * 32;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] = bf16_to_f32(src[i]);
        amax = fmaxf(amax, fabsf(v[i]));
    }
    int E = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;
    int eb = E - 2;
    eb = eb < -127 ? -127 : (eb > 127 ? 127 : eb);
    e8m0[b] = (uint8_t)(eb + 127);
    uint8_t *dst = q + n * (K / 2) + bb * 16;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        const uint32_t c0 = f32_to_e2m1(ldexpf(v[i], -eb));
        const uint32_t c1 = f32_to_e2m1(ldexpf(v[i + 1], -eb));
        dst[i / 2] = (uint8_t)(c0 | (c1 << 4));
    }
}

// Q4S (int4 codes on [-7, 7], fp32 scale per 64 columns): one thread per
// block.  s = fp32(amax / 7) and fp32(w / s) use the correctly rounded fp32
// division (this build keeps HIP's default), rint = round to nearest even.
__global__ void quant_q4s_kernel(const uint16_t *W, uint8_t *q, float *s, int64_t n_blocks, int K)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const int64_t nb_row = K / 64;
    const int64_t n = b / nb_row, bb = b % nb_row;
    const uint16_t *src = W + n * K + bb * 64;
    float amax = 0.f;
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(bf16_to_f32(src[i])));
    const float sc = amax / 7.0f;
    s[b] = amax == 0.f ? 0.f : sc;
    uint8_t *dst = q + n * (K / 2) + bb * 32;
    for (int i = 0; i < 64; i += 2) {
        int c[2] = {0, 0};
        if (amax != 0.f) {
            for (int j = 0; j < 2; ++j) {
                const float r = rintf(bf16_to_f32(src[i + j]) / sc);
                c[j] = (int)fminf(fmaxf(r, -7.f), 7.f);
            }
        }
        dst[i / 2] = (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
    }
}

// ----------------------------------------------------------------- argmax --
// Candidates of a grid-stride pass over x, one per block.
__global__ __launch_bounds__(K2_BLOCK) void argmax_kernel(const float *x, int n, ArgmaxArgs am)
{
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int i = blockIdx.x * K2_BLOCK + threadIdx.x; i < n; i += gridDim.x * K2_BLOCK)
        argmax_pair_max(bv, bi, x[i], i);
    argmax_block(bv, bi);
    if (threadIdx.x == 0) {
        am.part_v[blockIdx.x] = bv;
        am.part_i[blockIdx.x] = bi;
    }
}

// First maximum over the per-block candidates (value, then lowest index).
__global__ __launch_bounds__(K2_BLOCK) void argmax_final_kernel(ArgmaxArgs am, int n_blocks)
{
    // 16 candidates per thread loaded before the first comparison (one memory
    // round trip per 4096 blocks); the (greater value, then lower index) rule
    // gives the same winner in any order
    constexpr int AB = 16;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int b0 = 0; b0 < n_blocks; b0 += AB * K2_BLOCK) {
        float v[AB];
        int ix[AB];
#pragma unroll
        for (int u = 0; u < AB; ++u) {
            const int b = b0 + u * K2_BLOCK + (int)threadIdx.x;
            v[u] = b < n_blocks ? am.part_v[b] : -INFINITY;
            ix[u] = b < n_blocks ? am.part_i[b] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int u = 0; u < AB; ++u) argmax_pair_max(bv, bi, v[u], ix[u]);
    }
    argmax_block(bv, bi);
    if (threadIdx.x == 0) {
        *am.out_idx = bi;
        if (am.adv_pos) {
            const int p = *am.adv_pos;
            if (p >= 0 && p < am.adv_cap) *am.adv_pos = p + 1;
        }
    }
}

__global__ void pos_advance_kernel(int32_t *d_pos, int cap)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const int p = *d_pos;
        if (p >= 0 && p < cap) *d_pos = p + 1;
    }
}

int pos_advance_launch(int32_t *d_pos, int cap, hipStream_t st)
{
    hipLaunchKernelGGL(pos_advance_kernel, dim3(1), dim3(64), 0, st, d_pos, cap);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

int argmax_final_launch(const ArgmaxArgs &am, int n_blocks, hipStream_t st)
{
    hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(K2_BLOCK), 0, st, am, n_blocks);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// Streaming read of `blocks` contiguous slabs of n16 16-byte words each,
// with the decode GEMVs' load policy (non-temporal 128-bit loads, UNR loads
// per thread in flight, every address in range); one word per block goes to
// sink so that no load is dropped.
constexpr int READ_UNR = 8;
__global__ __launch_bounds__(K2_BLOCK) void read_probe_kernel(const k2_u4 *p, int64_t n16, uint32_t *sink)
{
    const k2_u4 *b = p + (int64_t)blockIdx.x * n16;
    uint32_t acc = 0u;
    for (int64_t i = threadIdx.x; i < n16; i += (int64_t)READ_UNR * K2_BLOCK) {
        k2_u4 v[READ_UNR];
#pragma unroll
        for (int d = 0; d < READ_UNR; ++d) {
            const int64_t j = i + (int64_t)d * K2_BLOCK;
            v[d] = __builtin_nontemporal_load(b + (j < n16 ? j : n16 - 1));
        }
#pragma unroll
        for (int d = 0; d < READ_UNR; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    acc = __builtin_amdgcn_readfirstlane(acc) ^ acc;
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

size_t argmax_ws_bytes()
{
    return k2_align256((size_t)K2_ARGMAX_MAX_BLOCKS * 4) * 2;
}

void argmax_ws_carve(void *ws, ArgmaxArgs &am)
{
    char *p = (char *)ws;
    am.part_v = (float *)p;
    p += k2_align256((size_t)K2_ARGMAX_MAX_BLOCKS * 4);
    am.part_i = (int *)p;
}

}  // namespace k2

using namespace k2;

// ---------------------------------------------------------------- C ABI --

extern "C" int k2_abi_version(void) { return K2_ABI_VERSION; }

extern "C" const char *k2_status_str(int status)
{
    switch (status) {
    case K2_OK: return "ok";
    case K2_EINVAL: return "invalid argument (null or misaligned pointer, bad size)";
    case K2_ERANGE: return "out of range (token, position or length)";
    case K2_EUNSUPPORTED: return "unsupported shape or dtype";
    case K2_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

int k2::rmsnorm_rows_launch(const float *x, const float *gamma, float *y, int rows, int hidden,
                            int groups, float eps, hipStream_t st)
{
    hipLaunchKernelGGL(rmsnorm_grouped_kernel, dim3(rows * groups), dim3(K2_BLOCK), 0, st, x, gamma, y,
                       hidden, groups, eps);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

int k2::rmsnorm_rows_planes_launch(const float *x, const float *gamma, uint16_t *yh, uint16_t *yl, int rows,
                                   int hidden, int groups, float eps, hipStream_t st)
{
    hipLaunchKernelGGL(rmsnorm_planes_kernel, dim3(rows * groups), dim3(K2_BLOCK), 0, st, x, gamma, yh, yl,
                       hidden, groups, eps);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" int k2_rmsnorm_grouped(const float *x, const float *gamma, float *y, int rows, int hidden,
                                  int groups, float eps, void *stream)
{
    if (!k2_ptr_ok(x) || !k2_ptr_ok(gamma) || !k2_ptr_ok(y)) return K2_EINVAL;
    if (rows <= 0 || hidden <= 0 || groups <= 0) return K2_EINVAL;
    if (hidden % groups) return K2_EUNSUPPORTED;
    hipLaunchKernelGGL(rmsnorm_grouped_kernel, dim3(rows * groups), dim3(K2_BLOCK), 0,
                       k2_stream(stream), x, gamma, y, hidden, groups, eps);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" int k2_rope_table(float *cos_sin, int cap, int head_dim, double theta, void *stream)
{
    if (!k2_ptr_ok(cos_sin)) return K2_EINVAL;
    if (cap <= 0 || head_dim <= 0 || head_dim % 2 || !(theta > 0)) return K2_EINVAL;
    const int64_t n = (int64_t)cap * (head_dim / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       k2_stream(stream), cos_sin, cap, head_dim, theta);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" int k2_rope(float *q, float *k, const float *cos_sin, int n_qh, int n_kv, int head_dim,
                       int pos, int cap, void *stream)
{
    if (!k2_ptr_ok(q) || !k2_ptr_ok(k) || !k2_ptr_ok(cos_sin)) return K2_EINVAL;
    if (n_qh <= 0 || n_kv <= 0 || cap <= 0) return K2_EINVAL;
    if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128) return K2_EUNSUPPORTED;
    if (pos < 0 || pos >= cap) return K2_ERANGE;
    const int n = (n_qh + n_kv) * (head_dim / 2);
    hipLaunchKernelGGL(rope_kernel, dim3((n + 255) / 256), dim3(256), 0, k2_stream(stream), q, k,
                       cos_sin, n_qh, n_kv, head_dim, pos);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" int k2_quantize_fp8_rows(const uint16_t *W, uint8_t *codes, float *row_scale, int N, int K,
                                    void *stream)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(codes) || !k2_ptr_ok(row_scale)) return K2_EINVAL;
    if (N <= 0 || K <= 0 || K % 16) return K2_EINVAL;
    hipLaunchKernelGGL(quant_fp8_rows_kernel, dim3(N), dim3(K2_BLOCK), 0, k2_stream(stream), W, codes,
                       row_scale, K);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" int k2_quantize_mxfp4(const uint16_t *W, uint8_t *q, uint8_t *e8m0, int N, int K,
                                 void *stream)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(q) || !e8m0) return K2_EINVAL;
    if (N <= 0 || K <= 0) return K2_EINVAL;
    if (K % 32) return K2_EUNSUPPORTED;
    const int64_t nb = (int64_t)N * (K / 32);
    hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                       k2_stream(stream), W, q, e8m0, nb, K);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" int k2_quantize_q4s(const uint16_t *W, uint8_t *q, float *s, int N, int K, void *stream)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(q) || !k2_ptr_ok(s)) return K2_EINVAL;
    if (N <= 0 || K <= 0) return K2_EINVAL;
    if (K % 64) return K2_EUNSUPPORTED;
    const int64_t nb = (int64_t)N * (K / 64);
    hipLaunchKernelGGL(quant_q4s_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                       k2_stream(stream), W, q, s, nb, K);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" size_t k2_argmax_workspace_bytes(int n) { return n > 0 ? argmax_ws_bytes() : 0; }

extern "C" int k2_argmax(const float *x, int n, int32_t *out_idx, void *ws, size_t ws_bytes,
                         void *stream)
{
    if (!k2_ptr_ok(x) || !out_idx || !ws || ((uintptr_t)ws & 255u)) return K2_EINVAL;
    if (n <= 0) return K2_EINVAL;
    if (ws_bytes < argmax_ws_bytes()) return K2_EINVAL;
    ArgmaxArgs am{};
    argmax_ws_carve(ws, am);
    am.out_idx = out_idx;
    int blocks = (n + K2_BLOCK - 1) / K2_BLOCK;
    if (blocks > 1024) blocks = 1024;
    am.n_blocks = blocks;
    hipLaunchKernelGGL(argmax_kernel, dim3(blocks), dim3(K2_BLOCK), 0, k2_stream(stream), x, n, am);
    K2_CHECK_LAUNCH();
    return argmax_final_launch(am, blocks, k2_stream(stream));
}

extern "C" int k2_read_probe(const void *buf, size_t bytes, int blocks, uint32_t *sink, void *stream)
{
    if (!k2_ptr_ok(buf) || !k2_ptr_ok(sink)) return K2_EINVAL;
    if (blocks <= 0 || bytes < (size_t)blocks * 16) return K2_EINVAL;
    const int64_t n16 = (int64_t)(bytes / 16 / (size_t)blocks);
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(K2_BLOCK), 0, k2_stream(stream),
                       (const k2_u4 *)buf, n16, sink);
    K2_CHECK_LAUNCH();
    return K2_OK;
}
