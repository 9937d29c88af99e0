// gemv.hip -- weight-streaming dequantizing GEMV for gfx950.
//
// y = W_hat x for the projections of the decode step ([k2-burn] "Model
// shape": QKV, O, SwiGLU gate/up, down, untied lm_head) with W stored as
// fp32, bf16, fp8 E4M3FN + per-row scale ([k2-burn] "Quantization") or MXFP4
// (E2M1 + E8M0 per 32 columns; [k3_run.c] header comment).
//
// Layout of the work:
//   * A 256-thread block stages the B activation vectors in LDS once
//     (optionally applying the grouped RMSNorm on the way in), then its four
//     waves stream rows.
//   * A wave owns R rows at a time (a "unit").  Lane l reads 16-byte chunk
//     c = l, l+64, ... of each of the R rows, so every load instruction of
//     the wave covers 1 KiB of contiguous weights, and the activation chunk
//     read from LDS is reused by the R rows.  U chunks per row are loaded
//     before any arithmetic so that R*U loads (R*U KiB per wave) are in
//     flight.
//   * Rows are reduced across the wave with butterfly shuffles; the epilogue
//     writes y (plus residual), or silu(gate) * up for row pairs, or a
//     (max, index) candidate for the argmax that follows the lm_head.
//   * Units are distributed grid-stride so the grid can be capped while
//     every unit is still covered.
// A 16-byte chunk holds 4 fp32, 8 bf16, 16 fp8 or 32 E2M1 values; for MXFP4
// a chunk is exactly one 32-column scale block, so the E8M0 scale is applied
// once to each chunk's partial sum.
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

template <int WDT> struct WT;
template <> struct WT<K2_F32>     { static constexpr int EPC = 4;  };
template <> struct WT<K2_BF16>    { static constexpr int EPC = 8;  };
template <> struct WT<K2_FP8E4M3> { static constexpr int EPC = 16; };
template <> struct WT<K2_MXFP4>   { static constexpr int EPC = 32; };

// dot of one 16-byte weight chunk with EPC consecutive activations in LDS
template <int WDT>
__device__ __forceinline__ float chunk_dot(const k2_u4 w, const float *__restrict__ x)
{
    float s0 = 0.f, s1 = 0.f;
    if constexpr (WDT == K2_F32) {
        const float4 xv = *reinterpret_cast<const float4 *>(x);
        s0 = __uint_as_float(w.x) * xv.x + __uint_as_float(w.y) * xv.y;
        s1 = __uint_as_float(w.z) * xv.z + __uint_as_float(w.w) * xv.w;
    } else if constexpr (WDT == K2_BF16) {
        const float4 a = *reinterpret_cast<const float4 *>(x);
        const float4 b = *reinterpret_cast<const float4 *>(x + 4);
        s0 = bf16_lo(w.x) * a.x + bf16_hi(w.x) * a.y;
        s1 = bf16_lo(w.y) * a.z + bf16_hi(w.y) * a.w;
        s0 += bf16_lo(w.z) * b.x + bf16_hi(w.z) * b.y;
        s1 += bf16_lo(w.w) * b.z + bf16_hi(w.w) * b.w;
    } else if constexpr (WDT == K2_FP8E4M3) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 xv = *reinterpret_cast<const float4 *>(x + 4 * i);
            const k2_f2 lo = fp8x2_lo(ws[i]);
            const k2_f2 hi = fp8x2_hi(ws[i]);
            s0 += lo.x * xv.x + lo.y * xv.y;
            s1 += hi.x * xv.z + hi.y * xv.w;
        }
    } else {  // MXFP4: 32 E2M1 values, low nibble first
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 xa = *reinterpret_cast<const float4 *>(x + 8 * i);
            const float4 xb = *reinterpret_cast<const float4 *>(x + 8 * i + 4);
            const k2_f2 v0 = fp4x2<0>(ws[i]);
            const k2_f2 v1 = fp4x2<1>(ws[i]);
            const k2_f2 v2 = fp4x2<2>(ws[i]);
            const k2_f2 v3 = fp4x2<3>(ws[i]);
            s0 += v0.x * xa.x + v0.y * xa.y;
            s1 += v1.x * xa.z + v1.y * xa.w;
            s0 += v2.x * xb.x + v2.y * xb.y;
            s1 += v3.x * xb.z + v3.y * xb.w;
        }
    }
    return s0 + s1;
}

// Stage B activation vectors [B][K] in LDS.  With PRO_NORM the single vector
// is the residual stream h and LDS receives GroupedRMSNorm(h) * gamma.
template <int B, int PRO>
__device__ __forceinline__ void stage_x(float *xs, const GemvArgs &a)
{
    const int K = a.K;
    if constexpr (PRO == PRO_NORM) {
        // B == 1.  Per-group sums of squares, then scale.
        __shared__ float red[K2_WAVES_PER_BLOCK][K2_MAX_GROUPS];
        const int G = a.groups, gs = K / G;
        float ss[K2_MAX_GROUPS];
#pragma unroll
        for (int g = 0; g < K2_MAX_GROUPS; ++g) ss[g] = 0.f;
        for (int i = threadIdx.x * 4; i < K; i += K2_BLOCK * 4) {
            const float4 v = *reinterpret_cast<const float4 *>(a.x + i);
            *reinterpret_cast<float4 *>(xs + i) = v;
            const int g = i / gs;   // gs % 4 == 0: a float4 never straddles groups
#pragma unroll
            for (int q = 0; q < K2_MAX_GROUPS; ++q)
                if (q == g) ss[q] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int g = 0; g < K2_MAX_GROUPS; ++g) {
            float t = wave_sum(ss[g]);
            if (lane == 0) red[wave][g] = t;
        }
        __syncthreads();
        __shared__ float rs[K2_MAX_GROUPS];
        if (threadIdx.x < G) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < K2_WAVES_PER_BLOCK; ++w) t += red[w][threadIdx.x];
            rs[threadIdx.x] = 1.0f / sqrtf(t / (float)gs + a.eps);
        }
        __syncthreads();
        for (int i = threadIdx.x * 4; i < K; i += K2_BLOCK * 4) {
            const float r = rs[i / gs];
            const float4 gm = *reinterpret_cast<const float4 *>(a.gamma + i);
            float4 v = *reinterpret_cast<float4 *>(xs + i);
            v.x = v.x * r * gm.x; v.y = v.y * r * gm.y;
            v.z = v.z * r * gm.z; v.w = v.w * r * gm.w;
            *reinterpret_cast<float4 *>(xs + i) = v;
        }
    } else {
        for (int i = threadIdx.x * 4; i < B * K; i += K2_BLOCK * 4)
            *reinterpret_cast<float4 *>(xs + i) = *reinterpret_cast<const float4 *>(a.x + i);
    }
    __syncthreads();
}

template <int WDT, int R, int U, int B, int PRO, int EPI>
__global__ __launch_bounds__(K2_BLOCK) void gemv_kernel(const GemvArgs a)
{
    extern __shared__ float4 lds4[];
    float *xs = reinterpret_cast<float *>(lds4);
    stage_x<B, PRO>(xs, a);

    constexpr int EPC = WT<WDT>::EPC;
    const int K = a.K;
    const int CPR = K / EPC;                       // 16-byte chunks per row
    const int64_t row_bytes = (int64_t)CPR * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const char *__restrict__ Wb = reinterpret_cast<const char *>(a.W);

    // argmax candidate of this thread (EPI_ARGMAX)
    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;

    for (int64_t unit = (int64_t)blockIdx.x * K2_WAVES_PER_BLOCK + wave; unit < a.n_units;
         unit += (int64_t)gridDim.x * K2_WAVES_PER_BLOCK) {
        int64_t rows[R];
        bool ok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (EPI == EPI_SWIGLU) {
                // first R/2 rows are gate rows, the next R/2 the matching up rows
                const int64_t g = unit * (R / 2) + (r % (R / 2));
                ok[r] = g < a.n_out;
                rows[r] = (r < R / 2) ? g : g + a.n_out;
            } else {
                rows[r] = unit * R + r;
                ok[r] = rows[r] < a.N;
            }
        }
        float acc[B][R];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[b][r] = 0.f;

        for (int c0 = 0; c0 < CPR; c0 += U * K2_WAVE) {
            k2_u4 w[U][R];
            float sc[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * K2_WAVE + lane;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (ok[r] && c < CPR) {
                        w[u][r] = __builtin_nontemporal_load(
                            reinterpret_cast<const k2_u4 *>(Wb + rows[r] * row_bytes) + c);
                        if constexpr (WDT == K2_MXFP4)
                            sc[u][r] = e8m0_to_f32(a.S8[rows[r] * CPR + c]);
                    } else {
                        w[u][r] = k2_u4{0u, 0u, 0u, 0u};
                        sc[u][r] = 0.f;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * K2_WAVE + lane;
                if (c < CPR) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float *xc = xs + b * K + c * EPC;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float d = chunk_dot<WDT>(w[u][r], xc);
                            if constexpr (WDT == K2_MXFP4) acc[b][r] += d * sc[u][r];
                            else acc[b][r] += d;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[b][r] = wave_sum(acc[b][r]);

        if constexpr (WDT == K2_FP8E4M3) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float s = ok[r] ? a.Sf[rows[r]] : 0.f;
#pragma unroll
                for (int b = 0; b < B; ++b) acc[b][r] *= s;
            }
        }

        if constexpr (EPI == EPI_SWIGLU) {
            // lane r' writes act[g] = silu(gate) * up
#pragma unroll
            for (int r = 0; r < R / 2; ++r) {
                if (lane == r && ok[r]) {
                    const float g = acc[0][r], u = acc[0][r + R / 2];
                    a.y[rows[r]] = g / (1.0f + expf(-g)) * u;
                }
            }
        } else if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (lane == r && ok[r]) {
                    const float v = acc[0][r];
                    a.y[rows[r]] = v;
                    if (v > best_v || (v == best_v && (int)rows[r] < best_i)) {
                        best_v = v;
                        best_i = (int)rows[r];
                    }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (lane == (b * R + r) % K2_WAVE && ok[r]) {
                        float v = acc[b][r];
                        if (a.residual) v += a.residual[(int64_t)b * a.N + rows[r]];
                        a.y[(int64_t)b * a.N + rows[r]] = v;
                    }
                }
        }
    }

    if constexpr (EPI == EPI_ARGMAX) argmax_block_finish(best_v, best_i, a.am);
}

// ------------------------------------------------------------------ host --

template <int WDT, int R, int U, int B, int PRO, int EPI>
static int launch(const GemvArgs &a0, hipStream_t st, int max_blocks)
{
    GemvArgs a = a0;
    const int64_t blocks_needed = (a.n_units + K2_WAVES_PER_BLOCK - 1) / K2_WAVES_PER_BLOCK;
    int blocks = (int)(blocks_needed < max_blocks ? blocks_needed : max_blocks);
    if (blocks < 1) blocks = 1;
    const size_t lds = (size_t)B * a.K * sizeof(float);
    if constexpr (EPI == EPI_ARGMAX) a.am.n_blocks = blocks;
    hipLaunchKernelGGL((gemv_kernel<WDT, R, U, B, PRO, EPI>), dim3(blocks), dim3(K2_BLOCK), lds,
                       st, a);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// Rows per unit and chunks per row in flight, by weight format: about
// R*U = 16 KiB of weights per wave in flight.
template <int WDT> struct Tile;
template <> struct Tile<K2_F32>     { static constexpr int R = 4, U = 4; };
template <> struct Tile<K2_BF16>    { static constexpr int R = 4, U = 4; };
template <> struct Tile<K2_FP8E4M3> { static constexpr int R = 8, U = 2; };
template <> struct Tile<K2_MXFP4>   { static constexpr int R = 8, U = 2; };

template <int WDT, int B, int PRO, int EPI>
static int gemv_tiled(GemvArgs a, hipStream_t st)
{
    // several activation vectors multiply the accumulators: fewer rows per unit
    constexpr int RB = (Tile<WDT>::R / B) > 1 ? Tile<WDT>::R / B : 1;
    constexpr int R = (EPI == EPI_SWIGLU) ? 2 * (Tile<WDT>::R / 2) : RB;
    if constexpr (EPI == EPI_SWIGLU) a.n_units = (a.n_out + R / 2 - 1) / (R / 2);
    else a.n_units = (a.N + R - 1) / R;
    return launch<WDT, R, Tile<WDT>::U, B, PRO, EPI>(a, st, K2_GEMV_MAX_BLOCKS);
}

int gemv_dispatch(int wdt, const GemvArgs &a, int pro, int epi, hipStream_t st)
{
#define K2_CASE(W)                                                                    \
    case W:                                                                           \
        if (pro == PRO_NONE && epi == EPI_PLAIN) {                                    \
            switch (a.B) {                                                            \
            case 1: return gemv_tiled<W, 1, PRO_NONE, EPI_PLAIN>(a, st);             \
            case 2: return gemv_tiled<W, 2, PRO_NONE, EPI_PLAIN>(a, st);             \
            case 4: return gemv_tiled<W, 4, PRO_NONE, EPI_PLAIN>(a, st);             \
            case 8: return gemv_tiled<W, 8, PRO_NONE, EPI_PLAIN>(a, st);             \
            default: return K2_EUNSUPPORTED;                                          \
            }                                                                         \
        }                                                                             \
        if (a.B != 1) return K2_EUNSUPPORTED;                                         \
        if (pro == PRO_NORM && epi == EPI_PLAIN) return gemv_tiled<W, 1, PRO_NORM, EPI_PLAIN>(a, st);   \
        if (pro == PRO_NORM && epi == EPI_SWIGLU) return gemv_tiled<W, 1, PRO_NORM, EPI_SWIGLU>(a, st); \
        if (pro == PRO_NORM && epi == EPI_ARGMAX) return gemv_tiled<W, 1, PRO_NORM, EPI_ARGMAX>(a, st); \
        return K2_EUNSUPPORTED;
    switch (wdt) {
        K2_CASE(K2_F32)
        K2_CASE(K2_BF16)
        K2_CASE(K2_FP8E4M3)
        K2_CASE(K2_MXFP4)
    default: return K2_EUNSUPPORTED;
    }
#undef K2_CASE
}

}  // namespace k2

using namespace k2;

// Generic entry points: B vectors (1, 2, 4 or 8; 3, 5..7 are padded by the
// caller-visible rule below), no prologue, optional residual.
static int gemv_entry(int wdt, const void *W, const void *S, const float *x, float *y,
                      const float *residual, int N, int K, int B, void *stream)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(x) || !k2_ptr_ok(y)) return K2_EINVAL;
    if (residual && !k2_aligned16(residual)) return K2_EINVAL;
    if (N <= 0 || K <= 0 || B <= 0) return K2_EINVAL;
    if ((wdt == K2_FP8E4M3 || wdt == K2_MXFP4) && !S) return K2_EINVAL;
    if (K % 32 != 0 || (int64_t)B * K > K2_MAX_LDS_FLOATS) return K2_EUNSUPPORTED;
    if (B != 1 && B != 2 && B != 4 && B != 8) return K2_EUNSUPPORTED;
    GemvArgs a{};
    a.W = W;
    a.Sf = (const float *)S;
    a.S8 = (const uint8_t *)S;
    a.x = x;
    a.y = y;
    a.residual = residual;
    a.N = N;
    a.K = K;
    a.B = B;
    return gemv_dispatch(wdt, a, PRO_NONE, EPI_PLAIN, k2_stream(stream));
}

extern "C" int k2_gemv_qbf16(const uint16_t *W, const float *x, float *y, const float *residual,
                             int N, int K, int B, void *stream)
{
    return gemv_entry(K2_BF16, W, nullptr, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_qfp8(const uint8_t *W, const float *row_scale, const float *x, float *y,
                            const float *residual, int N, int K, int B, void *stream)
{
    return gemv_entry(K2_FP8E4M3, W, row_scale, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_qmxfp4(const uint8_t *Wq, const uint8_t *We8m0, const float *x, float *y,
                              const float *residual, int N, int K, int B, void *stream)
{
    return gemv_entry(K2_MXFP4, Wq, We8m0, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_f32(const float *W, const float *x, float *y, const float *residual,
                           int N, int K, int B, void *stream)
{
    return gemv_entry(K2_F32, W, nullptr, x, y, residual, N, K, B, stream);
}

// Fused projection forms of the decode step, x = GroupedRMSNorm(h).
static int norm_gemv_check(int wdt, const void *W, const void *S, const float *h, const float *gamma,
                           int groups, const float *y, int N, int K)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(h) || !k2_ptr_ok(gamma) || !k2_ptr_ok(y)) return K2_EINVAL;
    if ((wdt == K2_FP8E4M3 || wdt == K2_MXFP4) && !S) return K2_EINVAL;
    if (N <= 0 || K <= 0 || groups <= 0) return K2_EINVAL;
    if (wdt != K2_F32 && wdt != K2_BF16 && wdt != K2_FP8E4M3 && wdt != K2_MXFP4) return K2_EUNSUPPORTED;
    if (K % 32 || K > K2_MAX_LDS_FLOATS || groups > K2_MAX_GROUPS || K % (4 * groups))
        return K2_EUNSUPPORTED;
    return K2_OK;
}

static GemvArgs norm_args(const void *W, const void *S, const float *h, const float *gamma, int groups,
                          float eps, float *y, int N, int K)
{
    GemvArgs a{};
    a.W = W;
    a.Sf = (const float *)S;
    a.S8 = (const uint8_t *)S;
    a.x = h;
    a.gamma = gamma;
    a.groups = groups;
    a.eps = eps;
    a.y = y;
    a.N = N;
    a.K = K;
    a.B = 1;
    return a;
}

extern "C" int k2_norm_gemv(k2_dtype wdt, const void *W, const void *S, const float *h,
                            const float *gamma, int groups, float eps, float *y, int N, int K,
                            void *stream)
{
    int rc = norm_gemv_check(wdt, W, S, h, gamma, groups, y, N, K);
    if (rc) return rc;
    return gemv_dispatch(wdt, norm_args(W, S, h, gamma, groups, eps, y, N, K), PRO_NORM, EPI_PLAIN,
                         k2_stream(stream));
}

extern "C" int k2_norm_gemv_swiglu(k2_dtype wdt, const void *W, const void *S, const float *h,
                                   const float *gamma, int groups, float eps, float *act, int inter,
                                   int K, void *stream)
{
    int rc = norm_gemv_check(wdt, W, S, h, gamma, groups, act, 2 * inter, K);
    if (rc) return rc;
    GemvArgs a = norm_args(W, S, h, gamma, groups, eps, act, 2 * inter, K);
    a.n_out = inter;
    return gemv_dispatch(wdt, a, PRO_NORM, EPI_SWIGLU, k2_stream(stream));
}

extern "C" int k2_norm_gemv_argmax(k2_dtype wdt, const void *W, const void *S, const float *h,
                                   const float *gamma, int groups, float eps, float *logits, int N,
                                   int K, int32_t *out_idx, void *ws, size_t ws_bytes, void *stream)
{
    int rc = norm_gemv_check(wdt, W, S, h, gamma, groups, logits, N, K);
    if (rc) return rc;
    if (!out_idx || !ws || ((uintptr_t)ws & 255u) || ws_bytes < argmax_ws_bytes()) return K2_EINVAL;
    GemvArgs a = norm_args(W, S, h, gamma, groups, eps, logits, N, K);
    argmax_ws_carve(ws, a.am);
    a.am.out_idx = out_idx;
    return gemv_dispatch(wdt, a, PRO_NORM, EPI_ARGMAX, k2_stream(stream));
}
