// dense_mfma.hip -- a bf16 weight matrix times a few fp32 activation rows
// (2 to 32 tokens at a time) on the matrix cores.
//
// The latent-MoE layer ([k3_run.c] forward(): router, W_dn, W_up and the
// shared experts) multiplies every dense matrix by T token rows.  With T rows
// a weight byte feeds 2T flops; past a few tokens that outgrows fp32 vector
// arithmetic, so here the product runs on v_mfma_f32_16x16x32_bf16:
//   * each activation is split into bf16 hi + bf16 lo (x - hi rounded again),
//     two MFMAs per weight tile, fp32 accumulation: the weights are exact in
//     bf16 and the split keeps ~16 bits of every activation;
//   * a block of 4 waves owns 256, 128 or 64 rows and one k-range (split-K); it stages
//     its slice of the activations once in LDS as the two bf16 planes, each
//     wave streams its 4, 2 or 1 row tiles of 16 rows from HBM, one 128-column chunk
//     ahead of the MFMAs;
//   * per-split partials [split][token][row] are summed in split order by a
//     second kernel, which also applies the epilogue (plain, add into y, or
//     SwiGLU of row pairs i, i + N/2) -- or, given arrival counters, by the
//     last block to finish of each row block (of each gate / up row-block
//     pair for SwiGLU): every block stores its partials at device scope and
//     counts itself, and the last one sums the group's partials in split
//     order (the same order, so the same result) and applies the epilogue.
//     That saves the second launch, whose gap and first-byte latency are
//     most of its cost at these sizes.
// Up to 16 tokens with K a multiple of 512 the weights take another route
// (dense_mfma_t_kernel): the operand layout puts 16 rows in every load
// instruction (64 bytes of each), which streams at ~3.6 TB/s where one row's
// contiguous 1 KiB per instruction streams at ~5.2 (same footprint, same
// loads in flight).  So each wave loads its 16 rows x 512 columns as 16 such
// row slices into registers and moves them into the operand layout through
// a 4 KiB LDS buffer, a quarter of the columns at a time.
// MFMA operand layout (16x16x32 bf16): lane l holds A row l % 16 and B column
// l % 16, elements k = 8 (l / 16) + [0, 8); D holds column l % 16, rows
// 4 (l / 16) + [0, 4).
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

typedef short dm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float dm_f32x4 __attribute__((ext_vector_type(4)));

constexpr int DM_WAVES = 4;                       // waves per block
constexpr int DM_MIN_ROWS = 16 * DM_WAVES;        // rows per block with one 16-row tile per wave
constexpr int DM_KC = 128;                        // columns per chunk (4 MFMA k-steps)
constexpr int DM_MAX_T = 32;                      // tokens per launch
constexpr int DM_FUSE_MAX = 128;                  // tokens x splits summed in-kernel at most

struct DenseArgs {
    const uint16_t *W;       // [N][K] bf16
    const float *x;          // [T][K] fp32
    float *part;             // [splits][TP][N]
    int N, K, T, KS;
    // in-kernel reduction (cnt non-null): arrival counters [groups], zero
    // between launches; the epilogue and its output y [T][N or N/2]
    unsigned *cnt;
    float *y;
    int epi;
    // optional grouped-RMSNorm prologue: x holds the residual stream h and
    // the product reads gamma * h / rms, the group's sum of squares given as
    // nsq [T][K / 64] partial sums over 64 consecutive elements
    const float *gamma, *nsq;
    int groups;
    float eps;
    // optional output osq [T][N / 64]: the partial sums of squares of the
    // final y rows (an epilogue that adds into the residual stream), the
    // nsq of the next product
    float *osq;
    // optional QKV epilogue (rope.qrot non-null): RoPE and the cache append
    DmRope rope;
};


__host__ __device__ constexpr int dm_lds_bytes(int tp, int ks) { return 2 * tp * (ks + 8) * 2; }

// Stage rows [0, NROW) of the activation slice x[.][k0, k0 + KS) in LDS as
// bf16 hi / lo planes of row stride RS (rows >= T are 0), in two steps: the
// loads (x, and for the norm prologue gamma and the sums of squares) are
// issued before the weight loads, so that the conversion waits for them
// alone (a wave's loads return in order) and overlaps the weights in flight.
template <int NROW, int KS>
struct DmX {
    static constexpr int NG = NROW * KS / 4 / 256;   // activation float4s per thread
    float4 xv[NG];
    float4 gm;                                    // gamma of the thread's 4 columns (the same in every g)
    float4 sq[2];                                 // float4s tid and tid + 256 of the (token, group) partials
};

template <int NROW, int KS>
__device__ __forceinline__ void dm_x_issue(const DenseArgs &a, DmX<NROW, KS> &s, int k0, int tid)
{
    constexpr int NG = DmX<NROW, KS>::NG;
    static_assert(256 % (KS / 4) == 0, "a thread's columns are the same in every row it stages");
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int i = g * 256 + tid, t = i / (KS / 4), k = (i % (KS / 4)) * 4;
        s.xv[g] = t < a.T ? *reinterpret_cast<const float4 *>(a.x + (int64_t)t * a.K + k0 + k)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (a.gamma) {
        s.gm = *reinterpret_cast<const float4 *>(a.gamma + k0 + (tid % (KS / 4)) * 4);
        // float4 j of the partials: (token, group) j / per4, its float4 j % per4
        const int per4 = a.K / a.groups / 256;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = tid + 256 * h, tg = j / per4, t = tg / a.groups;
            s.sq[h] = j < NROW * a.groups * per4 && t < a.T
                          ? reinterpret_cast<const float4 *>(a.nsq + (int64_t)t * (a.K / 64))[(tg % a.groups) * per4 +
                                                                                             j % per4]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

template <int NROW, int KS, int RS>
__device__ __forceinline__ void dm_x_finish(const DenseArgs &a, DmX<NROW, KS> &s, uint16_t *xh, uint16_t *xl,
                                            int k0, int tid)
{
    constexpr int NG = DmX<NROW, KS>::NG;
    if (a.gamma) {
        // 1 / rms of every (token, norm group) from its partials in order (the
        // same in every block), then h * r * gamma
        __shared__ float part4[512];
        __shared__ float rs[DM_MAX_T][K2_MAX_GROUPS];
        const int gs = a.K / a.groups, per4 = gs / 256;
        part4[tid] = (s.sq[0].x + s.sq[0].y) + (s.sq[0].z + s.sq[0].w);
        part4[tid + 256] = (s.sq[1].x + s.sq[1].y) + (s.sq[1].z + s.sq[1].w);
        __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the LDS store is done (weights stay in flight)
        __builtin_amdgcn_s_barrier();
        if (tid < NROW * a.groups) {
            float ss = 0.f;
            for (int i = 0; i < per4; ++i) ss += part4[tid * per4 + i];
            rs[tid / a.groups][tid % a.groups] = 1.0f / sqrtf(ss / (float)gs + a.eps);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int i = g * 256 + tid, t = i / (KS / 4), k = (i % (KS / 4)) * 4;
            const float r = rs[t][(k0 + k) / gs];
            s.xv[g] = make_float4(s.xv[g].x * r * s.gm.x, s.xv[g].y * r * s.gm.y, s.xv[g].z * r * s.gm.z,
                                  s.xv[g].w * r * s.gm.w);
        }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int i = g * 256 + tid, t = i / (KS / 4), k = (i % (KS / 4)) * 4;
        const float f[4] = {s.xv[g].x, s.xv[g].y, s.xv[g].z, s.xv[g].w};
        uint16_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = f32_to_bf16_rne(f[e]);
            l[e] = f32_to_bf16_rne(f[e] - bf16_to_f32(h[e]));
        }
        uint2 hv, lv;
        hv.x = h[0] | ((uint32_t)h[1] << 16); hv.y = h[2] | ((uint32_t)h[3] << 16);
        lv.x = l[0] | ((uint32_t)l[1] << 16); lv.y = l[2] | ((uint32_t)l[3] << 16);
        *reinterpret_cast<uint2 *>(xh + t * RS + k) = hv;
        *reinterpret_cast<uint2 *>(xl + t * RS + k) = lv;
    }
}

// The QKV product's last-block epilogue for a prefill chunk: the rows are
// heads of 128 (n_qh query heads, then n_kv keys, then n_kv values), two
// 64-row blocks each, counted together on counter h.  The last of the 2 x
// splits blocks of head h sums the head's partials in split order, rotates
// q and k by split-half RoPE at position pos0 + t (element d pairs with d +
// 64, held 16 lanes away), and writes q to qrot [T][n_qh][128] or k / v into
// the cache slot pos0 + t of their kv head in the cache format (int8: the
// head's absolute maximum / 127 as the scale, codes rounded to nearest even
// and clamped to +-127, the encoding of every other append).
template <int TP>
__device__ __forceinline__ void dm_reduce_rope(const DenseArgs &a, int tid)
{
    __shared__ int last;
    const int splits = gridDim.y, head = blockIdx.x / 2;
    __builtin_amdgcn_s_waitcnt(0);                // this thread's partial stores completed
    __syncthreads();
    if (tid == 0) {
        const unsigned arrivals = 2u * (unsigned)splits;
        const unsigned old = __hip_atomic_fetch_add(a.cnt + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == arrivals - 1;
        if (last) __hip_atomic_store(a.cnt + head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;

    const DmRope &r = a.rope;
    const int j = tid & 31;                       // rows 4j .. 4j+3 of the head
    const int n = head * 128 + 4 * j;
    const bool isq = head < r.n_qh, isk = !isq && head < r.n_qh + r.n_kv;
    const int g = isq ? 0 : isk ? head - r.n_qh : head - r.n_qh - r.n_kv;
    constexpr int B8 = 8;
    for (int t = tid / 32; t < a.T; t += 8) {
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < splits; s0 += B8) {
            float4 v[B8];
#pragma unroll
            for (int i = 0; i < B8; ++i)
                if (s0 + i < splits) v[i] = coh_load4(a.part, (int)(((int64_t)(s0 + i) * TP + t) * a.N + n));
#pragma unroll
            for (int i = 0; i < B8; ++i)
                if (s0 + i < splits) { sum.x += v[i].x; sum.y += v[i].y; sum.z += v[i].z; sum.w += v[i].w; }
        }
        float x[4] = {sum.x, sum.y, sum.z, sum.w};
        const int pos = r.pos0 + t;
        if (isq || isk) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __shfl_xor(x[e], 16);   // element d + 64 (d < 64) or d - 64
            const bool lo = j < 16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = (4 * j + e) & 63;
                const float c = r.cs[((int64_t)pos * 64 + i) * 2], sn = r.cs[((int64_t)pos * 64 + i) * 2 + 1];
                x[e] = lo ? x[e] * c - o[e] * sn : o[e] * sn + x[e] * c;
            }
        }
        if (isq) {
            *reinterpret_cast<float4 *>(r.qrot + ((int64_t)t * r.n_qh + head) * 128 + 4 * j) =
                make_float4(x[0], x[1], x[2], x[3]);
            continue;
        }
        const int64_t idx = ((int64_t)g * r.cap + pos) * 128 + 4 * j;
        if (r.kvdt == K2_F32) {
            *reinterpret_cast<float4 *>((float *)(isk ? r.kc : r.vc) + idx) = make_float4(x[0], x[1], x[2], x[3]);
        } else if (r.kvdt == K2_BF16) {
            uint2 b;
            b.x = f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
            b.y = f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
            *reinterpret_cast<uint2 *>((uint16_t *)(isk ? r.kc : r.vc) + idx) = b;
        } else {
            float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            const float sc = amax / 127.0f;
            uint32_t bits = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float q = 0.f;
                if (amax != 0.f) {
                    q = rintf(x[e] / sc);
                    q = fminf(fmaxf(q, -127.f), 127.f);
                }
                bits |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * e);
            }
            *reinterpret_cast<uint32_t *>((uint8_t *)(isk ? r.kc : r.vc) + idx) = bits;
            if (j == 0) (isk ? r.ks : r.vs)[(int64_t)g * r.cap + pos] = amax != 0.f ? sc : 0.f;
        }
    }
}

// After a block has stored its partials (at device scope): count its
// arrival; the last block of its group sums the group's partials in split
// order and applies the epilogue.  Row block b is a group alone, or for
// SwiGLU gate block b with up block b + rb / 2 (both counted on counter b).
template <int ROWS, int TP>
__device__ __forceinline__ void dm_reduce_last(const DenseArgs &a, int tid)
{
    __shared__ int last;
    const int rb = gridDim.x, splits = gridDim.y;
    const bool pair = a.epi == DM_EPI_SWIGLU;
    const int grp = pair ? blockIdx.x % (rb / 2) : blockIdx.x;
    const unsigned arrivals = (unsigned)(pair ? 2 * splits : splits);
    __builtin_amdgcn_s_waitcnt(0);                // this thread's partial stores completed
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == arrivals - 1;
        if (last) __hip_atomic_store(a.cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;

    // the group's outputs, each summed over the splits in split order: a
    // thread owns 4 consecutive outputs (gate rows for SwiGLU) of every
    // TSTEP-th token and loads 8 splits' partials before adding them
    constexpr int QUADS = ROWS / 4, TSTEP = 256 / QUADS;
    const int n_out = pair ? a.N / 2 : a.N;
    const int n = grp * ROWS + (tid % QUADS) * 4;
    // (with osq every thread stays to the end: the 16 threads holding 64
    // rows of a token add their squares across lanes)
    const bool have = n < n_out;
    if (!have && !a.osq) return;
    constexpr int B8 = 8;
    for (int t = tid / QUADS; t < a.T; t += TSTEP) {
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f), up = sum;
        for (int s0 = 0; have && s0 < splits; s0 += B8) {
            float4 v[B8], u[B8];
#pragma unroll
            for (int i = 0; i < B8; ++i) {
                if (s0 + i >= splits) break;
                const int o = (int)(((int64_t)(s0 + i) * TP + t) * a.N + n);
                v[i] = coh_load4(a.part, o);
                if (pair) u[i] = coh_load4(a.part, o + n_out);
            }
#pragma unroll
            for (int i = 0; i < B8; ++i) {
                if (s0 + i >= splits) break;
                sum.x += v[i].x; sum.y += v[i].y; sum.z += v[i].z; sum.w += v[i].w;
                if (pair) { up.x += u[i].x; up.y += u[i].y; up.z += u[i].z; up.w += u[i].w; }
            }
        }
        float4 *dst = reinterpret_cast<float4 *>(a.y + (int64_t)t * n_out + n);
        if (a.osq) {
            // the residual-stream form (ADD, N % 64 == 0): the new y and its
            // sum of squares over each 64 rows
            float ss = 0.f;
            if (have) {
                const float4 r = *dst;
                const float4 o = make_float4(r.x + sum.x, r.y + sum.y, r.z + sum.z, r.w + sum.w);
                *dst = o;
                ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
            }
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) ss += __shfl_xor(ss, d);
            if ((tid & 15) == 0 && have) a.osq[(int64_t)t * (a.N / 64) + n / 64] = ss;
        } else if (pair) {
            *dst = make_float4(sum.x / (1.0f + expf(-sum.x)) * up.x, sum.y / (1.0f + expf(-sum.y)) * up.y,
                               sum.z / (1.0f + expf(-sum.z)) * up.z, sum.w / (1.0f + expf(-sum.w)) * up.w);
        } else if (a.epi == DM_EPI_ADD) {
            const float4 r = *dst;
            *dst = make_float4(r.x + sum.x, r.y + sum.y, r.z + sum.z, r.w + sum.w);
        } else {
            *dst = sum;
        }
    }
}

template <int NTT, int KS, int RT>
__global__ __launch_bounds__(256) void dense_mfma_kernel(const DenseArgs a)
{
    constexpr int ROWS = RT * 16 * DM_WAVES;      // rows per block
    constexpr int TP = 16 * NTT;
    constexpr int RS = KS + 8;                    // LDS row stride (bf16): 16 B of pad per row
    constexpr int NCH = KS / DM_KC;               // chunks per split
    extern __shared__ float4 lds4[];
    uint16_t *xh = reinterpret_cast<uint16_t *>(lds4);
    uint16_t *xl = xh + TP * RS;
    const int split = blockIdx.y, k0 = split * KS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, c16 = lane & 15;

    // rows of this wave's tiles (tiles past N read the last tile again and
    // are never stored)
    int64_t rowoff[RT];
    bool rok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r0 = blockIdx.x * ROWS + (wave * RT + rt) * 16;
        rok[rt] = r0 < a.N;
        const int row = (rok[rt] ? r0 : a.N - 16) + c16;
        rowoff[rt] = (int64_t)row * a.K + k0 + q * 8;
    }
    const dm_bf16x8 *Wv = reinterpret_cast<const dm_bf16x8 *>(a.W);
    // chunk c of tile rt, k-step j: the 16 B at element rowoff + c*128 + 32j
    // (the 4 lanes of a row read 64 contiguous bytes per instruction)
    auto load_chunk = [&](int c, dm_bf16x8 (&w)[RT][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[rt][j] = __builtin_nontemporal_load(Wv + (rowoff[rt] + c * DM_KC + 32 * j) / 8);
    };
    DmX<TP, KS> xs;
    dm_x_issue<TP, KS>(a, xs, k0, tid);           // the activation slice's loads, then the weights'
    dm_bf16x8 wc[RT][4];
    load_chunk(0, wc);
    dm_x_finish<TP, KS, RS>(a, xs, xh, xl, k0, tid);   // as bf16 hi / lo planes, weights in flight
    __syncthreads();

    dm_f32x4 acc[RT][NTT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = dm_f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c, const dm_bf16x8 (&w)[RT][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = c * DM_KC + 32 * j + q * 8;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int t = tt * 16 + c16;
                const dm_bf16x8 bh = *reinterpret_cast<const dm_bf16x8 *>(xh + t * RS + kk);
                const dm_bf16x8 bl = *reinterpret_cast<const dm_bf16x8 *>(xl + t * RS + kk);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[rt][j], bh, acc[rt][tt], 0, 0, 0);
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[rt][j], bl, acc[rt][tt], 0, 0, 0);
                }
            }
        }
    };
    // one chunk ahead of the MFMAs; the last chunk without a next one
#pragma unroll 1
    for (int c = 0; c + 1 < NCH; ++c) {
        dm_bf16x8 wn[RT][4];
        load_chunk(c + 1, wn);
        compute(c, wc);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) wc[rt][j] = wn[rt][j];
    }
    compute(NCH - 1, wc);

    // partials: the lane holds rows 4q..4q+3 of each tile for token c16 + 16 tt
    // (device scope when another block sums them)
    const bool fuse = a.cnt != nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (!rok[rt]) continue;
        const int r0 = blockIdx.x * ROWS + (wave * RT + rt) * 16 + 4 * q;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = tt * 16 + c16;
            if (t >= a.T) continue;
            const int64_t o = ((int64_t)split * TP + t) * a.N + r0;
            const float4 v = make_float4(acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]);
            if (fuse) coh_store4(a.part, (int)o, v);
            else *reinterpret_cast<float4 *>(a.part + o) = v;
        }
    }
    if (!fuse) return;
    if constexpr (ROWS == 64) {
        if (a.rope.qrot) {
            dm_reduce_rope<TP>(a, tid);
            return;
        }
    }
    dm_reduce_last<ROWS, TP>(a, tid);
}

// Up to 16 tokens, K % 512 == 0: a block of 4 waves owns 64 rows and one
// 512-column split; wave w loads rows 16w .. 16w+15 one contiguous 1 KiB row
// slice per instruction (lane l: the row's 16-byte chunk l), then for each
// quarter p of the columns the lanes holding them (lanes 16p .. 16p+15)
// write their 16 rows into the wave's LDS buffer and the MFMAs read it back
// in the operand layout.  In the buffer, slot (c + r) % 16 of row r holds
// the quarter's chunk c, so that both the writes and the operand reads of
// 16 rows hit 16 different bank groups.  TM activation rows are staged (the
// operand's other token columns are zero).
constexpr int DT_KS = 512;
constexpr int DT_ROWS = 64;
__host__ __device__ constexpr int dt_lds_bytes(int tm) { return 2 * tm * (DT_KS + 8) * 2 + DM_WAVES * 4096; }

template <int TM>
__global__ __launch_bounds__(256) void dense_mfma_t_kernel(const DenseArgs a)
{
    constexpr int RS = DT_KS + 8;                 // activation row stride (bf16)
    extern __shared__ float4 lds4[];
    uint16_t *xh = reinterpret_cast<uint16_t *>(lds4);
    uint16_t *xl = xh + TM * RS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, c16 = lane & 15;
    char *tb = reinterpret_cast<char *>(xl + TM * RS) + wave * 4096;
    const int split = blockIdx.y, k0 = split * DT_KS;
    const int r0 = blockIdx.x * DT_ROWS + wave * 16;
    const bool rok = r0 < a.N;                    // a tile past N reads the last tile and stores nothing
    const int rl = rok ? r0 : a.N - 16;

    DmX<TM, DT_KS> xs;
    dm_x_issue<TM, DT_KS>(a, xs, k0, tid);        // the activation slice's loads, then the weights'
    k2_u4 w[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        w[r] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(a.W + (int64_t)(rl + r) * a.K + k0) + lane);
    dm_x_finish<TM, DT_KS, RS>(a, xs, xh, xl, k0, tid);
    __syncthreads();

    dm_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const dm_bf16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (p > 0) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the last quarter's reads are done
        if (q == p) {
#pragma unroll
            for (int r = 0; r < 16; ++r) *reinterpret_cast<k2_u4 *>(tb + r * 256 + ((c16 + r) & 15) * 16) = w[r];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * j + q;                  // the quarter's chunk of this lane's k group
            const dm_bf16x8 A = *reinterpret_cast<const dm_bf16x8 *>(tb + c16 * 256 + ((c + c16) & 15) * 16);
            dm_bf16x8 bh = zero, bl = zero;
            if (c16 < TM) {
                const int kk = (16 * p + c) * 8;
                bh = *reinterpret_cast<const dm_bf16x8 *>(xh + c16 * RS + kk);
                bl = *reinterpret_cast<const dm_bf16x8 *>(xl + c16 * RS + kk);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bl, acc, 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // partials [split][16][N]: the lane holds rows 4q .. 4q+3 for token c16
    const bool fuse = a.cnt != nullptr;
    if (rok && c16 < a.T) {
        const int64_t o = ((int64_t)split * 16 + c16) * a.N + r0 + 4 * q;
        const float4 v = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if (fuse) coh_store4(a.part, (int)o, v);
        else *reinterpret_cast<float4 *>(a.part + o) = v;
    }
    if (!fuse) return;
    if (a.rope.qrot) {
        dm_reduce_rope<16>(a, tid);
        return;
    }
    dm_reduce_last<DT_ROWS, 16>(a, tid);
}

// y[t][n] (+)= sum over splits in split order; SwiGLU: n < N/2 pairs rows n
// (gate) and n + N/2 (up) and y has N/2 columns.
// osq (ADD only, N % 64 == 0): the sums of squares of the new y over each
// 64 rows, one wave's worth.
__global__ __launch_bounds__(256) void dense_reduce_kernel(const float *part, int splits, int TP, int N,
                                                           int epi, float *y, float *osq)
{
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
    if (osq) {
        float ss = 0.f;
        if (n < n_out) {
            float s = 0.f;
            for (int sp = 0; sp < splits; ++sp) s += part[((int64_t)sp * TP + t) * N + n];
            float *dst = y + (int64_t)t * n_out + n;
            const float o = *dst + s;
            *dst = o;
            ss = o * o;
        }
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0 && n < n_out) osq[(int64_t)t * (N / 64) + n / 64] = ss;
        return;
    }
    if (n >= n_out) return;
    float s = 0.f, u = 0.f;
    for (int sp = 0; sp < splits; ++sp) {
        const float *p = part + ((int64_t)sp * TP + t) * N;
        s += p[n];
        if (epi == DM_EPI_SWIGLU) u += p[n + n_out];
    }
    float *dst = y + (int64_t)t * n_out + n;
    if (epi == DM_EPI_SWIGLU) *dst = s / (1.0f + expf(-s)) * u;
    else if (epi == DM_EPI_ADD) *dst += s;
    else *dst = s;
}

// Tile shape: 16-row tiles per wave (RT: 256, 128 or 64 rows per block) and
// columns per split (KS), the first of (4, 1024), (2, 1024), (1, 1024) (up
// to 16 tokens: with 32 their activation slice fills the LDS of a compute
// unit, and measured slower), (4, 512), (2, 512), (1, 512), (1, 256),
// (1, 128) that divides K and gives at least 256 blocks (else the last): the
// longest splits first (their chunks stream one ahead of the
// matrix cores, and fewer splits leave fewer partials), then the largest row
// blocks (an activation fragment read from LDS feeds RT row tiles).
struct DmTile { int rt, ks; };
static DmTile dm_tile(int N, int K, int T)
{
    static const DmTile cand[] = {{4, 1024}, {2, 1024}, {1, 1024}, {4, 512}, {2, 512},
                                  {1, 512},  {1, 256},  {1, 128}};
    const int tp = (T < DM_MAX_T ? T : DM_MAX_T) <= 16 ? 16 : 32;
    for (const DmTile &c : cand) {
        if (c.ks == 1024 && tp > 16) continue;
        const int64_t rb = (N + c.rt * DM_MIN_ROWS - 1) / (c.rt * DM_MIN_ROWS);
        if (K % c.ks == 0 && rb * (K / c.ks) >= 256) return c;
    }
    return {1, DM_KC};
}

bool dense_mfma_ok(int N, int K) { return N >= 16 && N % 16 == 0 && K % DM_KC == 0; }

// The row-slice form: up to 16 tokens and K a multiple of 512, for tall
// products (16384 rows and more) and for those of 2^24 weights and more
// whose T x splits partial rows are summed in the last blocks.  Measured per
// launch in 8-token verification rounds at the 3.7B shape: gate/up (20480 x
// 2560) 26.4 against 32.6 us, lm_head 208 against 292 us; but QKV (6144 x
// 2560) 13.5 against 12.0, O (2560 x 4096) 13.2 against 10.6, and down
// (2560 x 10240, 20 splits: a second launch sums them) 23.8 against 18.9.
static bool dt_ok(int N, int K, int T)
{
    if (T > 16 || K % DT_KS) return false;
    return N >= 16384 || ((int64_t)N * K >= (int64_t)1 << 24 && (int64_t)T * (K / DT_KS) <= DM_FUSE_MAX);
}

size_t dense_mfma_ws_bytes(int N, int K, int T)
{
    if (!dense_mfma_ok(N, K) || T < 2) return 0;
    if (dt_ok(N, K, T)) return (size_t)(K / DT_KS) * 16 * N * 4;
    const int tp = (T < DM_MAX_T ? T : DM_MAX_T) <= 16 ? 16 : 32;
    return (size_t)(K / dm_tile(N, K, T).ks) * tp * N * 4;
}

int dense_mfma_cnt_words(int N) { return (N + DM_MIN_ROWS - 1) / DM_MIN_ROWS; }

template <int NTT, int KS>
static void dm_go(int rt, dim3 grid, size_t lds, hipStream_t st, const DenseArgs &a)
{
    if (rt == 4) hipLaunchKernelGGL((dense_mfma_kernel<NTT, KS, 4>), grid, dim3(256), lds, st, a);
    else if (rt == 2) hipLaunchKernelGGL((dense_mfma_kernel<NTT, KS, 2>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((dense_mfma_kernel<NTT, KS, 1>), grid, dim3(256), lds, st, a);
}

// y = W x for T token rows (T >= 2), through per-split partials in `part`
// (dense_mfma_ws_bytes); groups of up to 32 tokens run one after another.
// cnt (nullable, dense_mfma_cnt_words(N) zeroed words, left zero): sum the
// partials in the product's last blocks instead of a second launch (SwiGLU
// only when N / 2 is a multiple of the row block).  nrm: the grouped
// RMSNorm applied to x on the way in (x the residual stream, nrm.nsq its
// 64-element sums of squares); osq (ADD only): those sums of the new y.
bool dense_norm_ok(int hidden, int groups)
{
    // whole float4s of 64-element partials per group, at most two per thread of a block
    return groups >= 1 && groups <= K2_MAX_GROUPS && hidden % groups == 0 && (hidden / groups) % 256 == 0 &&
           (int64_t)DM_MAX_T * hidden / 256 <= 512;
}

int dense_mfma(const uint16_t *W, const float *x, float *y, int N, int K, int T, int epi, float *part,
               hipStream_t st, unsigned *cnt, const DmNorm &nrm, float *osq, const DmRope *rope)
{
    if (!dense_mfma_ok(N, K) || T < 2) return K2_EUNSUPPORTED;
    if (nrm.gamma && (!nrm.nsq || !dense_norm_ok(K, nrm.groups))) return K2_EINVAL;
    if (osq && (epi != DM_EPI_ADD || N % 64)) return K2_EINVAL;
    if (rope) {
        // the QKV epilogue runs in the last blocks of 64-row blocks only:
        // refused (nothing enqueued) where the product would take another form
        if (epi != DM_EPI_PLAIN || !cnt || N % 128 || N != (rope->n_qh + 2 * rope->n_kv) * 128) return K2_EINVAL;
        const int splits = dt_ok(N, K, T) ? K / DT_KS : K / dm_tile(N, K, T).ks;
        if (T > DM_MAX_T || (!dt_ok(N, K, T) && dm_tile(N, K, T).rt != 1) || (int64_t)T * splits > DM_FUSE_MAX)
            return K2_EUNSUPPORTED;
    }
    const DmRope rp = rope ? *rope : DmRope{};
    const int n_out_all = epi == DM_EPI_SWIGLU ? N / 2 : N;
    if (dt_ok(N, K, T)) {
        const int splits = K / DT_KS;
        if (epi == DM_EPI_SWIGLU && (N / 2) % DT_ROWS) cnt = nullptr;
        if ((int64_t)T * splits > DM_FUSE_MAX) cnt = nullptr;
        DenseArgs a{W, x, part, N, K, T, DT_KS, cnt, y, epi, nrm.gamma, nrm.nsq, nrm.groups, nrm.eps, osq, rp};
        const dim3 grid((N + DT_ROWS - 1) / DT_ROWS, splits);
        if (T <= 4) hipLaunchKernelGGL(dense_mfma_t_kernel<4>, grid, dim3(256), dt_lds_bytes(4), st, a);
        else if (T <= 8) hipLaunchKernelGGL(dense_mfma_t_kernel<8>, grid, dim3(256), dt_lds_bytes(8), st, a);
        else hipLaunchKernelGGL(dense_mfma_t_kernel<16>, grid, dim3(256), dt_lds_bytes(16), st, a);
        K2_CHECK_LAUNCH();
        if (cnt) return K2_OK;
        hipLaunchKernelGGL(dense_reduce_kernel, dim3((n_out_all + 255) / 256, T), dim3(256), 0, st, part, splits,
                           16, N, epi, y, osq);
        K2_CHECK_LAUNCH();
        return K2_OK;
    }
    const DmTile tile = dm_tile(N, K, T);
    const int KS = tile.ks, splits = K / KS, rows = tile.rt * DM_MIN_ROWS;
    const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
    if (epi == DM_EPI_SWIGLU && (N / 2) % rows) cnt = nullptr;
    // the last block of a group reads T x splits partial rows: past ~128 of
    // them that tail costs more than the second launch (3.7B shape,
    // verification rounds with every product fused: T = 2 3.90 against 4.23
    // ms, T = 8 4.85 against 4.84, T = 16 5.85 against 5.12)
    if ((int64_t)(T < DM_MAX_T ? T : DM_MAX_T) * splits > DM_FUSE_MAX) cnt = nullptr;
    for (int t0 = 0; t0 < T; t0 += DM_MAX_T) {
        const int tg = T - t0 < DM_MAX_T ? T - t0 : DM_MAX_T;
        DenseArgs a{W, x + (int64_t)t0 * K, part, N, K, tg, KS, cnt, y + (int64_t)t0 * n_out, epi, nrm.gamma,
                    nrm.nsq ? nrm.nsq + (int64_t)t0 * (K / 64) : nullptr, nrm.groups, nrm.eps,
                    osq ? osq + (int64_t)t0 * (N / 64) : nullptr, rp};
        const dim3 grid((N + rows - 1) / rows, splits);
        const int tp = tg <= 16 ? 16 : 32;
        const size_t lds = dm_lds_bytes(tp, KS);
        if (tp == 16) {
            if (KS == 1024) dm_go<1, 1024>(tile.rt, grid, lds, st, a);
            else if (KS == 512) dm_go<1, 512>(tile.rt, grid, lds, st, a);
            else if (KS == 256) dm_go<1, 256>(tile.rt, grid, lds, st, a);
            else dm_go<1, 128>(tile.rt, grid, lds, st, a);
        } else {
            if (KS == 1024) dm_go<2, 1024>(tile.rt, grid, lds, st, a);
            else if (KS == 512) dm_go<2, 512>(tile.rt, grid, lds, st, a);
            else if (KS == 256) dm_go<2, 256>(tile.rt, grid, lds, st, a);
            else dm_go<2, 128>(tile.rt, grid, lds, st, a);
        }
        K2_CHECK_LAUNCH();
        if (cnt) continue;
        hipLaunchKernelGGL(dense_reduce_kernel, dim3((n_out + 255) / 256, tg), dim3(256), 0, st, part,
                           splits, tp, N, epi, y + (int64_t)t0 * n_out, a.osq);
        K2_CHECK_LAUNCH();
    }
    return K2_OK;
}

}  // namespace k2
