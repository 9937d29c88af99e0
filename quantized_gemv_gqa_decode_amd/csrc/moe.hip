// moe.hip -- routed-expert MXFP4 GEMV of a latent-MoE layer, gathered by
// expert, and the composite layer around it.
//
// The layer ([k3_run.c] real_cfg_hardcoded(): 896 experts, top-16, 2 shared,
// latent 3584, inter 3072, routed_scale, renorm, latent_norm;
// [cpu_weights.rs] MoeWeights: down, up, norm, router, bias, experts (w1, w2,
// w3), shared), for each of T independent token rows x [hidden]:
//   sigma = sigmoid(W_r x); sel = top-k of sigma + bias (the bias selects
//   only); g_j = routed_scale * sigma_sel_j / sum of the selected sigma;
//   z = RMSNorm(W_dn x); r = sum_j g_j W2_e(silu(W1_e z) * (W3_e z));
//   y = W_up r + sum_s W2_s(silu(W1_s x) * (W3_s x)).
// Routed experts are MXFP4 ([k3_run.c] header: the routed experts are
// multiplied directly from their MXFP4 storage); the dense parts are bf16.
//
// Gather by expert: the P = T*k (token, slot) pairs are bucketed by expert
// (a stable counting sort, so the order is fixed); the weights of each
// selected expert are streamed once for all of its tokens (in groups of TB
// staged in LDS); the per-pair outputs are then combined in slot order.  No
// float atomics: the result is the same from run to run.
#include <mutex>

#include "gemv_impl.h"

namespace k2 {

constexpr int MOE_R = 4;           // rows per wave unit (W13: 2 gate + 2 up rows)
constexpr int MOE_U = 2;           // 16-byte chunks per lane per pass
constexpr int MOE_NU = 4;          // units per wave
constexpr int MOE_MAX_K = 4096;    // latent and inter bound (LDS and x registers)
constexpr int MOE_MAX_PAIRS = 1024;
constexpr int MOE_MAX_EXPERTS = 1024;

struct MoeWs {
    int *sorted_tok;               // [P] token of the i-th pair in bucket order
    int *pair_index;               // [P] bucket position of pair p = t*k + slot (-1: dropped)
    int *item_e, *item_off, *item_cnt;  // [P] work items: expert, first position, tokens (<= TB)
    int *n_items;                  // [1]
    float *act;                    // [P][inter] silu(W1 z) * (W3 z), bucket order
    float *out;                    // [P][latent] W2 act, bucket order
};

static size_t moe_ws_layout(int T, int top_k, int inter, int latent, MoeWs *w, void *base)
{
    const size_t P = (size_t)T * top_k;
    size_t off = 0;
    char *b = (char *)base;
    auto take = [&](size_t bytes) {
        char *p = b ? b + off : nullptr;
        off += k2_align256(bytes);
        return p;
    };
    char *st = take(P * 4), *pi = take(P * 4);
    char *ie = take(P * 4), *io = take(P * 4), *ic = take(P * 4), *ni = take(4);
    char *act = take(P * inter * 4), *out = take(P * latent * 4);
    if (w) {
        w->sorted_tok = (int *)st; w->pair_index = (int *)pi;
        w->item_e = (int *)ie; w->item_off = (int *)io; w->item_cnt = (int *)ic;
        w->n_items = (int *)ni; w->act = (float *)act; w->out = (float *)out;
    }
    return off;
}

// ------------------------------------------------------------------ route --
// One block per token: sigma = sigmoid(logit); the top_k experts by
// sigma + bias in descending order, the lower index first on equal scores
// (top_k rounds of a block argmax); gates renormalised over the selected
// sigma and scaled by routed_scale.
// (value, index) first maximum across the wave, in every lane: DPP inside
// rows, then lane swaps across rows and halves (VALU only; the order in
// which pairs meet does not matter for a maximum with an index tie-break).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true); }
__device__ __forceinline__ void argmax_wave_valu(float &v, int &i)
{
    argmax_pair_max(v, i, dpp<0xB1>(v), dpp_i<0xB1>(i));     // quad_perm [1,0,3,2]
    argmax_pair_max(v, i, dpp<0x4E>(v), dpp_i<0x4E>(i));     // quad_perm [2,3,0,1]
    argmax_pair_max(v, i, dpp<0x141>(v), dpp_i<0x141>(i));   // row_half_mirror
    argmax_pair_max(v, i, dpp<0x140>(v), dpp_i<0x140>(i));   // row_mirror
    auto r16v = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    auto r16i = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
    v = __uint_as_float(r16v[0]); i = (int)r16i[0];
    argmax_pair_max(v, i, __uint_as_float(r16v[1]), (int)r16i[1]);
    auto r32v = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    auto r32i = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
    v = __uint_as_float(r32v[0]); i = (int)r32i[0];
    argmax_pair_max(v, i, __uint_as_float(r32v[1]), (int)r32i[1]);
}

__global__ __launch_bounds__(K2_WAVE) void moe_route_kernel(const float *logits, const float *bias,
                                                            int n_experts, int top_k,
                                                            float routed_scale, int32_t *topk_idx,
                                                            float *topk_w)
{
    // one wave per token: lane l keeps experts l, l + 64, ... in registers;
    // every round is a lane-local first maximum plus a wave (value, index)
    // reduction, with no barriers
    constexpr int RPL = MOE_MAX_EXPERTS / K2_WAVE;
    __shared__ float sel_sig[32];
    const int t = blockIdx.x, lane = threadIdx.x;
    float sc[RPL], sg[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int e = lane + K2_WAVE * i;
        sc[i] = -INFINITY;
        sg[i] = 0.f;
        if (e < n_experts) {
            const float l = logits[(int64_t)t * n_experts + e];
            sg[i] = 1.0f / (1.0f + expf(-l));
            sc[i] = sg[i] + (bias ? bias[e] : 0.f);
        }
    }
    for (int j = 0; j < top_k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < RPL; ++i)               // increasing expert id: ties keep the lower
            if (sc[i] > bv) { bv = sc[i]; bi = lane + K2_WAVE * i; }
        argmax_wave_valu(bv, bi);                   // the same (value, index) in every lane
        bi = __builtin_amdgcn_readfirstlane(bi);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            if (lane + K2_WAVE * i == bi) { s = sg[i]; sc[i] = -INFINITY; }
        s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), bi % K2_WAVE));
        if (lane == 0) {
            topk_idx[(int64_t)t * top_k + j] = bi;
            sel_sig[j] = s;
        }
    }
    __syncthreads();
    if (lane == 0) {
        float tot = 0.f;
        for (int j = 0; j < top_k; ++j) tot += sel_sig[j];
        for (int j = 0; j < top_k; ++j) topk_w[(int64_t)t * top_k + j] = routed_scale * sel_sig[j] / tot;
    }
}

// ----------------------------------------------------------------- bucket --
// One block: stable counting sort of the P pairs by expert.  Pair p with
// expert e_p goes to position #{q : e_q < e_p} + #{q < p : e_q == e_p}.  The
// pairs of one expert (c of them) then form ceil(c / TB) work items of at
// most TB consecutive pairs; items are numbered in expert order.  An id
// outside [0, n_experts) sets *d_err and its pair is dropped (pair_index -1).
__global__ __launch_bounds__(1024) void moe_bucket_kernel(const int32_t *topk_idx, int P, int top_k,
                                                          int n_experts, int TB, MoeWs w,
                                                          int32_t *d_err)
{
    constexpr int BAD = 0x7FFFFFFF;
    __shared__ int4 ex4[MOE_MAX_PAIRS / 4];
    __shared__ int4 groups4[MOE_MAX_PAIRS / 4];   // items of the expert at its first pair, else 0
    __shared__ int n_items;
    int *ex = reinterpret_cast<int *>(ex4);
    int *groups = reinterpret_cast<int *>(groups4);
    const int p = threadIdx.x;
    const int P4 = (P + 3) / 4;                   // scans read 4 pairs at a time; the pad is BAD
    if (p == 0) n_items = 0;
    int e = BAD;
    if (p < P) {
        e = topk_idx[p];
        if (e < 0 || e >= n_experts) {
            if (d_err) *d_err = K2_ERANGE;
            e = BAD;
        }
    }
    if (p < 4 * P4) {
        ex[p] = e;
        groups[p] = 0;
    }
    __syncthreads();
    int idx = 0, same = 0, g = 0;
    if (p < P) {
        int less = 0, before = 0;
#pragma unroll 8
        for (int q4 = 0; q4 < P4; ++q4) {
            const int4 f = ex4[q4];
            const int q = 4 * q4;
            less += (f.x < e) + (f.y < e) + (f.z < e) + (f.w < e);
            same += (f.x == e) + (f.y == e) + (f.z == e) + (f.w == e);
            before += ((q < p) & (f.x == e)) + ((q + 1 < p) & (f.y == e)) + ((q + 2 < p) & (f.z == e)) +
                      ((q + 3 < p) & (f.w == e));
        }
        idx = less + before;
        g = (before == 0 && e != BAD) ? (same + TB - 1) / TB : 0;
        w.sorted_tok[idx] = p / top_k;
        w.pair_index[p] = e == BAD ? -1 : idx;
        groups[p] = g;
    }
    __syncthreads();
    if (g > 0) {
        int base = 0;
#pragma unroll 8
        for (int q4 = 0; q4 < P4; ++q4) {
            const int4 f = ex4[q4], gr = groups4[q4];
            base += (f.x < e ? gr.x : 0) + (f.y < e ? gr.y : 0) + (f.z < e ? gr.z : 0) + (f.w < e ? gr.w : 0);
        }
        for (int i = 0; i < g; ++i) {
            const int left = same - i * TB;
            w.item_e[base + i] = e;
            w.item_off[base + i] = idx + i * TB;
            w.item_cnt[base + i] = left < TB ? left : TB;
        }
        atomicAdd(&n_items, g);
    }
    __syncthreads();
    if (p == 0) *w.n_items = n_items;
}

// -------------------------------------------------------------- expert GEMV --
// Block (x, u): row block x of the u-th selected expert.  Its tokens are taken
// TB at a time; their input vectors are staged in LDS (permuted layout of
// gemv_impl.h) and every weight chunk loaded serves all of them.  A wave runs
// MOE_NU units of MOE_R rows; the next unit's loads are issued before the
// current unit is reduced.
//   UP:   W13 = [W1 (inter rows); W3 (inter rows)] of the expert, K = latent;
//         unit = 2 gate rows + the 2 matching up rows; writes
//         act[pair][i] = silu(gate_i) * up_i.  x rows: z[token].
//   DOWN: W2 [latent][inter], K = inter; writes out[pair][row].  x rows:
//         act[pair] (the pairs of an expert are contiguous).
template <bool UP>
struct MoeRows {
    __device__ static void get(int64_t unit, int n_out, int N, int64_t *rows, bool *ok)
    {
#pragma unroll
        for (int r = 0; r < MOE_R; ++r) {
            if constexpr (UP) {
                const int64_t g = unit * (MOE_R / 2) + (r % (MOE_R / 2));
                ok[r] = g < n_out;
                rows[r] = (r < MOE_R / 2) ? g : g + n_out;
            } else {
                rows[r] = unit * MOE_R + r;
                ok[r] = rows[r] < N;
            }
        }
    }
};

__device__ __forceinline__ void moe_load(const uint8_t *Wq, const uint8_t *Ws, const int64_t *rows,
                                         int N, int p, int CPR, int lane,
                                         k2_u4 (&wv)[MOE_U][MOE_R], float (&sc)[MOE_U][MOE_R])
{
    const int64_t row_bytes = (int64_t)CPR * 16;
#pragma unroll
    for (int uu = 0; uu < MOE_U; ++uu) {
        const int c = (p * MOE_U + uu) * K2_WAVE + lane;
        const int cc = c < CPR ? c : CPR - 1;
#pragma unroll
        for (int r = 0; r < MOE_R; ++r) {
            const int64_t rr = rows[r] < N ? rows[r] : N - 1;
            wv[uu][r] = __builtin_nontemporal_load(
                reinterpret_cast<const k2_u4 *>(Wq + rr * row_bytes) + cc);
            sc[uu][r] = e8m0_to_f32(Ws[rr * CPR + cc]);
        }
    }
}

// The units of one wave for an item of exactly NB tokens (a compile-time
// count: no per-token branches inside the unrolled dot).  wv/sc hold the
// first unit's pass-0 loads on entry.
template <bool UP, int NB>
__device__ __forceinline__ void moe_units(const uint8_t *Wq, const uint8_t *Wsc, const float *xs,
                                          int N, int n_out, int CPR, int S, int passes,
                                          int64_t unit0, int lane, int off, float *dst,
                                          int64_t (&rows)[MOE_R], bool (&ok)[MOE_R],
                                          k2_u4 (&wv)[MOE_U][MOE_R], float (&sc)[MOE_U][MOE_R])
{
    constexpr int EPC = 32;
#pragma unroll 1
    for (int iu = 0; iu < MOE_NU; ++iu) {
        float acc[NB][MOE_R];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < MOE_R; ++r) acc[b][r] = 0.f;
#pragma unroll 1
        for (int p = 0; p < passes; ++p) {
            if (p > 0) moe_load(Wq, Wsc, rows, N, p, CPR, lane, wv, sc);
#pragma unroll
            for (int uu = 0; uu < MOE_U; ++uu) {
                const int c = (p * MOE_U + uu) * K2_WAVE + lane;
                if (c < CPR)
                    chunk_rows<K2_MXFP4, MOE_R, NB>(wv[uu], sc[uu], xs + c * 4, 4 * S, EPC * S, NB,
                                                    acc);
            }
        }
        int64_t cur_rows[MOE_R];
        bool cur_ok[MOE_R];
#pragma unroll
        for (int r = 0; r < MOE_R; ++r) { cur_rows[r] = rows[r]; cur_ok[r] = ok[r]; }
        if (iu + 1 < MOE_NU) {                     // uniform
            MoeRows<UP>::get(unit0 + (int64_t)(iu + 1) * K2_WAVES_PER_BLOCK, n_out, N, rows, ok);
            moe_load(Wq, Wsc, rows, N, 0, CPR, lane, wv, sc);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < MOE_R; ++r) acc[b][r] = wave_sum(acc[b][r]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (UP) {
                float *o = dst + (int64_t)(off + b) * n_out;
#pragma unroll
                for (int r = 0; r < MOE_R / 2; ++r)
                    if (lane == b * MOE_R + r && cur_ok[r]) {
                        const float g = acc[b][r], v = acc[b][r + MOE_R / 2];
                        o[cur_rows[r]] = g / (1.0f + expf(-g)) * v;
                    }
            } else {
                float *o = dst + (int64_t)(off + b) * N;
#pragma unroll
                for (int r = 0; r < MOE_R; ++r)
                    if (lane == b * MOE_R + r && cur_ok[r]) o[cur_rows[r]] = acc[b][r];
            }
        }
    }
}

template <bool UP, int TB>
__global__ __launch_bounds__(K2_BLOCK) __attribute__((amdgpu_waves_per_eu(4, 8)))
void moe_expert_kernel(const float *xsrc, const uint8_t *wq, const uint8_t *ws, int N, int K,
                       int n_out, MoeWs w, float *dst)
{
    constexpr int EPC = 32;
    constexpr int XV = TB * MOE_MAX_K / (4 * K2_BLOCK);   // float4 staging loads per thread
    extern __shared__ float4 lds4[];
    float *xs = reinterpret_cast<float *>(lds4);
    const int item = blockIdx.y;
    if (item >= *w.n_items) return;                // block-uniform, before any barrier
    const int e = w.item_e[item], off = w.item_off[item], tb = w.item_cnt[item];
    const int CPR = K / EPC;
    const int S = xs_plane(CPR);
    const int passes = (CPR + MOE_U * K2_WAVE - 1) / (MOE_U * K2_WAVE);
    const uint8_t *Wq = wq + (int64_t)e * N * CPR * 16;
    const uint8_t *Wsc = ws + (int64_t)e * N * CPR;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t unit0 = (int64_t)blockIdx.x * (K2_WAVES_PER_BLOCK * MOE_NU) + wave;

    // activations of the item's tokens (clamped, unconditional loads) ...
    float4 xr[XV];
    const int n = tb * K;
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int i = (v * K2_BLOCK + threadIdx.x) * 4;
        const int ii = i < n ? i : 0;
        const int b = ii / K, k = ii - b * K;
        const int64_t src = UP ? w.sorted_tok[off + b] : off + b;
        xr[v] = *reinterpret_cast<const float4 *>(xsrc + src * K + k);
    }
    // ... then the first unit's weights
    int64_t rows[MOE_R];
    bool ok[MOE_R];
    k2_u4 wv[MOE_U][MOE_R];
    float sc[MOE_U][MOE_R];
    MoeRows<UP>::get(unit0, n_out, N, rows, ok);
    moe_load(Wq, Wsc, rows, N, 0, CPR, lane, wv, sc);
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int i = (v * K2_BLOCK + threadIdx.x) * 4;
        if (i < n) {
            const int b = i / K, k = i - b * K;
            *reinterpret_cast<float4 *>(xs + b * EPC * S + xs_offset<EPC>(k, S)) = xr[v];
        }
    }
    __syncthreads();
    if (TB == 1 || tb == 1)                        // uniform
        moe_units<UP, 1>(Wq, Wsc, xs, N, n_out, CPR, S, passes, unit0, lane, off, dst, rows, ok, wv, sc);
    else
        moe_units<UP, TB>(Wq, Wsc, xs, N, n_out, CPR, S, passes, unit0, lane, off, dst, rows, ok, wv, sc);
}

// r[t][j] = sum over slots s in order of topk_w[t][s] * out[pair_index[t][s]][j]
// (the slots' indices, weights and rows are loaded 16 at a time before the
// first is added: one memory round trip per 16 slots)
__global__ void moe_combine_kernel(const float *topk_w, int top_k, int latent, MoeWs w, float *r)
{
    const int t = blockIdx.y;
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= latent) return;
    constexpr int SB = 16;
    float acc = 0.f;
    for (int s0 = 0; s0 < top_k; s0 += SB) {
        int idx[SB];
        float wt[SB], v[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            idx[i] = s0 + i < top_k ? w.pair_index[t * top_k + s0 + i] : -1;
            wt[i] = s0 + i < top_k ? topk_w[t * top_k + s0 + i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < SB; ++i) v[i] = idx[i] >= 0 ? w.out[(int64_t)idx[i] * latent + j] : 0.f;
#pragma unroll
        for (int i = 0; i < SB; ++i)
            if (idx[i] >= 0) acc += wt[i] * v[i];
    }
    r[(int64_t)t * latent + j] = acc;
}

// act[t][i] = silu(gu[t][i]) * gu[t][inter + i]
__global__ void swiglu_rows_kernel(const float *gu, int inter, float *act)
{
    const int t = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= inter) return;
    const float g = gu[(int64_t)t * 2 * inter + i], u = gu[(int64_t)t * 2 * inter + inter + i];
    act[(int64_t)t * inter + i] = g / (1.0f + expf(-g)) * u;
}

__global__ void add_rows_kernel(float *y, const float *a, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] += a[i];
}

template <bool UP, int TB>
static int moe_expert_go(const float *x, const uint8_t *wq, const uint8_t *ws, int N, int K,
                         int n_out, const MoeWs &w, float *dst, int max_u, hipStream_t st)
{
    const int64_t units = UP ? (n_out + MOE_R / 2 - 1) / (MOE_R / 2) : (N + MOE_R - 1) / MOE_R;
    const int per_block = K2_WAVES_PER_BLOCK * MOE_NU;
    const int bx = (int)((units + per_block - 1) / per_block);
    const size_t lds = (size_t)TB * 32 * xs_plane(K / 32) * sizeof(float);
    hipLaunchKernelGGL((moe_expert_kernel<UP, TB>), dim3(bx, max_u), dim3(K2_BLOCK), lds, st, x, wq,
                       ws, N, K, n_out, w, dst);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// tokens of one expert per work item (weight pass): one for a single-token
// call, else two (an expert rarely holds more than two of a few dozen
// tokens, and a small LDS footprint keeps more blocks resident)
static int moe_tb(int T) { return T == 1 ? 1 : 2; }

int moe_expert_launch(const float *z, int T, int latent, int inter, const int32_t *topk_idx,
                      const float *topk_w, int top_k, int n_experts, const uint8_t *w13q,
                      const uint8_t *w13s, const uint8_t *w2q, const uint8_t *w2s, float *r,
                      int32_t *d_err, void *ws, hipStream_t st)
{
    MoeWs w;
    moe_ws_layout(T, top_k, inter, latent, &w, ws);
    const int P = T * top_k;
    const int TB = moe_tb(T);
    hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(MOE_MAX_PAIRS), 0, st, topk_idx, P, top_k,
                       n_experts, TB, w, d_err);
    K2_CHECK_LAUNCH();
    const int max_u = P;                           // items <= pairs
    int rc;
    if (TB == 1) {
        if ((rc = moe_expert_go<true, 1>(z, w13q, w13s, 2 * inter, latent, inter, w, w.act, max_u, st)))
            return rc;
        if ((rc = moe_expert_go<false, 1>(w.act, w2q, w2s, latent, inter, 0, w, w.out, max_u, st)))
            return rc;
    } else {
        if ((rc = moe_expert_go<true, 2>(z, w13q, w13s, 2 * inter, latent, inter, w, w.act, max_u, st)))
            return rc;
        if ((rc = moe_expert_go<false, 2>(w.act, w2q, w2s, latent, inter, 0, w, w.out, max_u, st)))
            return rc;
    }
    hipLaunchKernelGGL(moe_combine_kernel, dim3((latent + 255) / 256, T), dim3(256), 0, st, topk_w,
                       top_k, latent, w, r);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// bf16 GEMV of T token rows, as many rows per launch as the staged
// activations allow (1, 2, 4 or 8)
static int gemv_rows_bf16(const uint16_t *W, const float *x, float *y, int N, int K, int T,
                          hipStream_t st, const float *residual = nullptr)
{
    const int bmax = K2_MAX_LDS_FLOATS / K;
    int t = 0;
    while (t < T) {
        const int left = T - t < bmax ? T - t : bmax;
        const int b = left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1;
        GemvArgs a{};
        a.W = W;
        a.x = x + (int64_t)t * K;
        a.y = y + (int64_t)t * N;
        a.N = N;
        a.K = K;
        a.B = b;
        a.residual = residual ? residual + (int64_t)t * N : nullptr;
        const int rc = gemv_dispatch(K2_BF16, a, PRO_NONE, EPI_PLAIN, st);
        if (rc) return rc;
        t += b;
    }
    return K2_OK;
}

// Partials of the matrix-core path for the layer's dense products at T rows.
static size_t moe_dense_part_bytes(const k2_moe_config *c, int T)
{
    size_t m = dense_mfma_ws_bytes(c->n_experts, c->hidden, T);
    const size_t o[4] = {dense_mfma_ws_bytes(c->latent, c->hidden, T),
                         dense_mfma_ws_bytes(c->hidden, c->latent, T),
                         dense_mfma_ws_bytes(2 * c->inter, c->hidden, T),
                         dense_mfma_ws_bytes(c->hidden, c->inter, T)};
    for (size_t v : o) m = v > m ? v : m;
    return m;
}

// y (+)= W x for T rows of bf16 weights: the matrix cores for T >= 2 when
// the shape allows, else the GEMV (rows staged 1, 2, 4 or 8 at a time)
// followed by the epilogue kernel.
static int dense_rows_bf16(const uint16_t *W, const float *x, float *y, int N, int K, int T, int epi,
                           float *part, float *tmp, hipStream_t st)
{
    if (T >= 2 && dense_mfma_ok(N, K)) return dense_mfma(W, x, y, N, K, T, epi, part, st);
    if (epi == DM_EPI_PLAIN) return gemv_rows_bf16(W, x, y, N, K, T, st);
    if (epi == DM_EPI_ADD) return gemv_rows_bf16(W, x, y, N, K, T, st, y);   // y = W x + y in one launch
    int rc = gemv_rows_bf16(W, x, tmp, N, K, T, st);
    if (rc) return rc;
    if (epi == DM_EPI_SWIGLU) {
        hipLaunchKernelGGL(swiglu_rows_kernel, dim3((N / 2 + 255) / 256, T), dim3(256), 0, st, tmp, N / 2, y);
    } else {
        const int64_t n = (int64_t)T * N;
        hipLaunchKernelGGL(add_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y, tmp, n);
    }
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// A second stream per device for the work that reads only the layer input
// (the router, the shared experts): it runs beside the latent / routed-expert
// chain.  Created once per device (default priority) and kept for the life
// of the process, with its fork, routing and join events; calls of
// k2_moe_layer that overlap in time on one device would share them and must
// not (as they must not share a workspace).
struct MoeSide {
    hipStream_t s;
    hipEvent_t fork, routed, join;
};
constexpr int MOE_MAX_DEVICES = 64;
static std::mutex g_moe_side_mu;
static MoeSide g_moe_side[MOE_MAX_DEVICES];
static bool g_moe_side_ok[MOE_MAX_DEVICES];

// The side stream of the current device, created on first use -- but not
// while `st` is being captured into a graph (creating a stream could end the
// capture): the layer then runs on `st` alone.
static MoeSide *moe_side(hipStream_t st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MOE_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_moe_side_mu);
    if (!g_moe_side_ok[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
        MoeSide m{};
        if (hipStreamCreateWithFlags(&m.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&m.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&m.routed, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&m.join, hipEventDisableTiming) != hipSuccess)
            return nullptr;
        g_moe_side[dev] = m;
        g_moe_side_ok[dev] = true;
    }
    return &g_moe_side[dev];
}

static int moe_dims_check(int T, int latent, int inter, int top_k, int n_experts)
{
    if (T <= 0 || latent <= 0 || inter <= 0 || top_k <= 0 || n_experts <= 0) return K2_EINVAL;
    if (latent % 32 || inter % 32 || latent > MOE_MAX_K || inter > MOE_MAX_K) return K2_EUNSUPPORTED;
    if (top_k > 32 || top_k > n_experts || n_experts > MOE_MAX_EXPERTS) return K2_EUNSUPPORTED;
    if ((int64_t)T * top_k > MOE_MAX_PAIRS) return K2_EUNSUPPORTED;
    return K2_OK;
}

static bool ws_ok(const void *ws, size_t have, size_t need)
{
    return ws && !((uintptr_t)ws & 255u) && have >= need;
}

}  // namespace k2

using namespace k2;

extern "C" size_t k2_moe_route_workspace_bytes(int T, int n_experts)
{
    if (T <= 0 || n_experts <= 0) return 0;
    return k2_align256((size_t)T * n_experts * 4);
}

extern "C" int k2_moe_route(const uint16_t *Wr, const float *bias, const float *x, int T,
                            int hidden, int n_experts, int top_k, float routed_scale,
                            int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                            void *stream)
{
    if (!k2_ptr_ok(Wr) || !k2_ptr_ok(x) || !topk_idx || !topk_w) return K2_EINVAL;
    if (T <= 0 || hidden <= 0 || n_experts <= 0 || top_k <= 0) return K2_EINVAL;
    if (hidden % 32 || hidden > K2_MAX_LDS_FLOATS || n_experts > MOE_MAX_EXPERTS || top_k > 32 ||
        top_k > n_experts)
        return K2_EUNSUPPORTED;
    if (!ws_ok(ws, ws_bytes, k2_moe_route_workspace_bytes(T, n_experts))) return K2_EINVAL;
    hipStream_t st = k2_stream(stream);
    float *logits = (float *)ws;
    const int rc = gemv_rows_bf16(Wr, x, logits, n_experts, hidden, T, st);
    if (rc) return rc;
    hipLaunchKernelGGL(moe_route_kernel, dim3(T), dim3(K2_WAVE), 0, st, logits, bias, n_experts,
                       top_k, routed_scale, topk_idx, topk_w);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

extern "C" size_t k2_moe_workspace_bytes(int T, int top_k, int latent, int inter)
{
    if (T <= 0 || top_k <= 0 || inter <= 0 || latent <= 0) return 0;
    return moe_ws_layout(T, top_k, inter, latent, nullptr, nullptr);
}

extern "C" int k2_moe_expert_gemv(const float *z, int T, int latent, int inter,
                                  const int32_t *topk_idx, const float *topk_w, int top_k,
                                  int n_experts, const uint8_t *w13q, const uint8_t *w13s,
                                  const uint8_t *w2q, const uint8_t *w2s, float *r, int32_t *d_err,
                                  void *ws, size_t ws_bytes, void *stream)
{
    if (!k2_ptr_ok(z) || !topk_idx || !topk_w || !k2_ptr_ok(w13q) || !w13s || !k2_ptr_ok(w2q) ||
        !w2s || !k2_ptr_ok(r))
        return K2_EINVAL;
    const int rc = moe_dims_check(T, latent, inter, top_k, n_experts);
    if (rc) return rc;
    if (!ws_ok(ws, ws_bytes, k2_moe_workspace_bytes(T, top_k, latent, inter))) return K2_EINVAL;
    return moe_expert_launch(z, T, latent, inter, topk_idx, topk_w, top_k, n_experts, w13q, w13s,
                             w2q, w2s, r, d_err, ws, k2_stream(stream));
}

// ----------------------------------------------------------- whole layer --

extern "C" size_t k2_moe_layer_workspace_bytes(const k2_moe_config *c, int T)
{
    if (!c || T <= 0 || c->top_k <= 0 || c->n_experts <= 0 || c->latent <= 0 || c->inter <= 0 ||
        c->hidden <= 0)
        return 0;
    size_t n = 0;
    n += k2_align256((size_t)T * c->n_experts * 4);                 // router logits
    n += k2_align256((size_t)T * c->top_k * 4) * 2;                 // topk idx, gates
    n += k2_align256((size_t)T * c->latent * 4) * 2;                // z, r
    n += k2_align256((size_t)T * 2 * c->inter * 4);                 // shared gate/up
    n += k2_align256((size_t)T * c->inter * 4);                     // shared act
    n += k2_align256((size_t)T * c->hidden * 4);                    // shared out
    n += k2_align256(moe_dense_part_bytes(c, T)) * 2;               // matrix-core partials (both streams)
    n += moe_ws_layout(T, c->top_k, c->inter, c->latent, nullptr, nullptr);
    return n;
}

extern "C" int k2_moe_layer(const k2_moe_layer_weights *w, const float *x, int T, float *y,
                            int32_t *topk_idx_out, float *topk_w_out, int32_t *d_err, void *ws,
                            size_t ws_bytes, void *stream)
{
    if (!w || !k2_ptr_ok(x) || !k2_ptr_ok(y)) return K2_EINVAL;
    const k2_moe_config *c = &w->cfg;
    int rc = moe_dims_check(T, c->latent, c->inter, c->top_k, c->n_experts);
    if (rc) return rc;
    if (c->hidden <= 0) return K2_EINVAL;
    if (c->hidden % 32 || c->hidden > K2_MAX_LDS_FLOATS) return K2_EUNSUPPORTED;
    if (c->n_shared < 0 || (c->n_shared > 0 && (!k2_ptr_ok(w->sh_w13) || !k2_ptr_ok(w->sh_w2))))
        return K2_EINVAL;
    if (!k2_ptr_ok(w->w_router) || !k2_ptr_ok(w->w_down) || !k2_ptr_ok(w->latent_gamma) ||
        !k2_ptr_ok(w->w_up) || !k2_ptr_ok(w->w13q) || !w->w13s || !k2_ptr_ok(w->w2q) || !w->w2s)
        return K2_EINVAL;
    if (!ws_ok(ws, ws_bytes, k2_moe_layer_workspace_bytes(c, T))) return K2_EINVAL;
    hipStream_t st = k2_stream(stream);
    char *p = (char *)ws;
    auto take = [&](size_t bytes) { char *q = p; p += k2_align256(bytes); return q; };
    float *logits = (float *)take((size_t)T * c->n_experts * 4);
    int32_t *tidx = (int32_t *)take((size_t)T * c->top_k * 4);
    float *tw = (float *)take((size_t)T * c->top_k * 4);
    float *z = (float *)take((size_t)T * c->latent * 4);
    float *r = (float *)take((size_t)T * c->latent * 4);
    float *sgu = (float *)take((size_t)T * 2 * c->inter * 4);
    float *sact = (float *)take((size_t)T * c->inter * 4);
    float *sout = (float *)take((size_t)T * c->hidden * 4);
    float *part = (float *)take(moe_dense_part_bytes(c, T));
    float *part2 = (float *)take(moe_dense_part_bytes(c, T));
    void *ews = p;

    // Two streams.  The library's side stream takes the work that reads only
    // the layer input: the router (its routing is waited for before the
    // routed experts), then the shared experts, y = sum_s W2_s(silu(W1_s x) *
    // (W3_s x)) (waited for before W_up adds into y).  The caller's stream
    // runs W_dn, the latent norm, the routed experts and W_up.  Without a
    // side stream everything runs on the caller's stream in the same order.
    MoeSide *side = moe_side(st);
    const hipStream_t ss = side ? side->s : st;
    if (side && (hipEventRecord(side->fork, st) != hipSuccess || hipStreamWaitEvent(ss, side->fork, 0) != hipSuccess))
        return K2_EHIP;
    if ((rc = dense_rows_bf16(w->w_router, x, logits, c->n_experts, c->hidden, T, DM_EPI_PLAIN, part2, nullptr,
                              ss)))
        return rc;
    hipLaunchKernelGGL(moe_route_kernel, dim3(T), dim3(K2_WAVE), 0, ss, logits, w->router_bias,
                       c->n_experts, c->top_k, c->routed_scale, tidx, tw);
    K2_CHECK_LAUNCH();
    if (side && hipEventRecord(side->routed, ss) != hipSuccess) return K2_EHIP;
    for (int s = 0; s < c->n_shared; ++s) {
        const uint16_t *w13 = w->sh_w13 + (int64_t)s * 2 * c->inter * c->hidden;
        const uint16_t *w2 = w->sh_w2 + (int64_t)s * c->hidden * c->inter;
        if ((rc = dense_rows_bf16(w13, x, sact, 2 * c->inter, c->hidden, T, DM_EPI_SWIGLU, part2, sgu, ss)))
            return rc;
        if ((rc = dense_rows_bf16(w2, sact, y, c->hidden, c->inter, T, s == 0 ? DM_EPI_PLAIN : DM_EPI_ADD, part2,
                                  sout, ss)))
            return rc;
    }
    if (side && hipEventRecord(side->join, ss) != hipSuccess) return K2_EHIP;

    // latent: z = RMSNorm(W_dn x)
    if ((rc = dense_rows_bf16(w->w_down, x, z, c->latent, c->hidden, T, DM_EPI_PLAIN, part, nullptr, st)))
        return rc;
    if ((rc = k2_rmsnorm_grouped(z, w->latent_gamma, z, T, c->latent, 1, c->eps, stream))) return rc;
    // routed experts, once the routing is in
    if (side && hipStreamWaitEvent(st, side->routed, 0) != hipSuccess) return K2_EHIP;
    if ((rc = moe_expert_launch(z, T, c->latent, c->inter, tidx, tw, c->top_k, c->n_experts, w->w13q,
                                w->w13s, w->w2q, w->w2s, r, d_err, ews, st)))
        return rc;
    // y (+)= W_up r, after the side stream's work
    if (side && hipStreamWaitEvent(st, side->join, 0) != hipSuccess) return K2_EHIP;
    if ((rc = dense_rows_bf16(w->w_up, r, y, c->hidden, c->latent, T, c->n_shared > 0 ? DM_EPI_ADD : DM_EPI_PLAIN,
                              part, sout, st)))
        return rc;
    if (topk_idx_out) {
        if (hipMemcpyAsync(topk_idx_out, tidx, (size_t)T * c->top_k * 4, hipMemcpyDeviceToDevice, st))
            return K2_EHIP;
    }
    if (topk_w_out) {
        if (hipMemcpyAsync(topk_w_out, tw, (size_t)T * c->top_k * 4, hipMemcpyDeviceToDevice, st))
            return K2_EHIP;
    }
    return K2_OK;
}
