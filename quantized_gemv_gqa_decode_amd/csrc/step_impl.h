// step_impl.h -- the whole decode position as ONE persistent kernel.
//
// The multi-kernel step pays a fixed start-up and drain cost per kernel
// (a few microseconds each, about 180 kernels per position).  Here a single
// cooperative launch runs every phase of the position, in order:
//   embed | per layer: QKV (norm prologue) | RoPE + KV append + split-K
//   attention (the last block of a kv head combines its splits) | O +
//   residual | gate/up (norm prologue) + SwiGLU | down + residual |
//   final norm + lm_head + argmax (the last block reduces the block
//   candidates in block order).
// Phases are separated by a grid barrier.  Weights do not depend on the
// activations, so before arriving at a barrier every wave issues the loads
// of its first unit of the NEXT phase: the barrier's latency overlaps HBM
// traffic instead of idling it.
//
// Activations move between blocks that may sit on different XCDs, whose L2
// caches are not coherent with each other.  Every activation vector of the
// launch has its own address (a per-layer "trail": qkv, attention output,
// residual after O, SwiGLU output, residual after down), written once with
// device-scope (write-through) stores that complete before the writer's
// block arrives at the next barrier.  Readers then use ordinary loads: a
// line written in this launch cannot be stale in any L2, because no block
// read that address earlier in the launch, and caches are invalidated
// between launches.  (Reading with device-scope loads instead sends every
// block to memory for the same few kilobytes at the same moment.)  The
// attention partials are reused by every layer and are read at device
// scope.  The KV cache slot written at `pos` is read back only from LDS
// inside the launch.
//
// Each wave issues its next-phase loads after its stores have completed and
// before the barrier.  (Thread 0's barrier atomics wait behind its wave's
// loads, since a wave observes memory in issue order; the loads of the whole
// grid are in flight meanwhile.)
//
// Barriers count up from zero within a launch (the host clears the sync
// words with a fill kernel before each launch).  Every spin is bounded: a
// block that waits too long sets a sticky abort word, reports K2_EHIP in
// d_err, and every block then leaves the kernel at its next barrier, so the
// grid always drains.
#pragma once
#include "attn_impl.h"
#include "gemv_impl.h"

namespace k2 {

constexpr int STEP_SPIN_LIMIT = 1 << 17;     // polls per barrier (each ~1 us)
constexpr int STEP_GROUPS = 8;               // first-level barrier groups
constexpr int SYNC_STRIDE = 64;              // words between sync counters (256 B)
// sync word layout (unsigned [STEP_SYNC_WORDS])
constexpr int SYNC_GRP = 0;                                  // [8] group arrival counters
constexpr int SYNC_GLOB = SYNC_GRP + STEP_GROUPS * SYNC_STRIDE;  // global arrival counter
constexpr int SYNC_GEN = SYNC_GLOB + SYNC_STRIDE;            // [8] released barrier count
constexpr int SYNC_ABORT = SYNC_GEN + STEP_GROUPS * SYNC_STRIDE;
constexpr int SYNC_AM = SYNC_ABORT + SYNC_STRIDE;            // argmax arrivals
constexpr int SYNC_HEAD = SYNC_AM + SYNC_STRIDE;             // [n_kv] attention split arrivals
constexpr int STEP_MAX_KV = 64;
constexpr int STEP_SYNC_WORDS = SYNC_HEAD + STEP_MAX_KV * SYNC_STRIDE;

// Tiles (rows per wave unit R, 16-byte chunks per lane per pass U) of the
// five projections, per weight format: QKV, O, gate/up, down, lm_head.
template <int WDT> struct StepTiles;
template <> struct StepTiles<K2_F32>     { static constexpr int RQ = 2, UQ = 2, RO = 1, UO = 2, RG = 2, UG = 2, RD = 1, UD = 2, RL = 2, UL = 2; };
// Sized for the 3.7B shape (hidden 2560, 32x128 heads, inter 10240) so that
// with ~2048 waves every wave's share of QKV, O and down is one unit whose
// loads are all issued before the barrier; gate/up streams a few units.
template <> struct StepTiles<K2_BF16>    { static constexpr int RQ = 4, UQ = 5, RO = 2, UO = 10, RG = 4, UG = 5, RD = 1, UD = 20, RL = 4, UL = 5; };
template <> struct StepTiles<K2_FP8E4M3> { static constexpr int RQ = 4, UQ = 3, RO = 2, UO = 4, RG = 4, UG = 3, RD = 1, UD = 10, RL = 4, UL = 3; };
template <> struct StepTiles<K2_MXFP4>   { static constexpr int RQ = 4, UQ = 2, RO = 2, UO = 2, RG = 4, UG = 2, RD = 1, UD = 5, RL = 4, UL = 2; };

struct StepArgs {
    const k2_layer *layers;      // device copy of the layer table
    const void *embed;
    const void *lm, *lm_s;
    const float *g_final, *rope;
    float *trail;                        // h0, then per layer [qkv | o | hA | act | hB]
    int64_t layer_floats;                // per-layer stride of the trail
    int off_qkv, off_o, off_ha, off_act, off_hb;   // offsets in a layer's slice
    float *logits;                       // nullable: no head
    float *part, *part_ml;               // attention partials
    float *am_v;                         // argmax block candidates [grid]
    int *am_i;
    int32_t *next;                       // argmax output (nullable)
    const int32_t *d_token;              // nullable: use token
    int32_t *d_err;                      // nullable
    unsigned *sync;                      // STEP_SYNC_WORDS, zero at launch
    int token, pos, len;
    int n_layers, H, inter, vocab, groups, n_qh, n_kv, cap;
    int embdt;
    int attn_S, attn_chunk;
    float eps, scale;
};

// Optional phase trace for performance work (never enabled in the library
// build): block 0 records the 100 MHz real-time counter when it arrives at
// and leaves every barrier.
#ifdef K2_STEP_TRACE
static __device__ unsigned long long k2_step_trace[2048];
#define K2_TRACE(i)                                                                     \
    do {                                                                                \
        if (blockIdx.x == 0 && (i) < 2048) k2_step_trace[i] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define K2_TRACE(i) \
    do {        \
    } while (0)
#endif

__device__ __forceinline__ unsigned sync_add(unsigned *p)
{
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned sync_load(const unsigned *p)
{
    return __hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void sync_store(unsigned *p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier number `bar` (1, 2, ...; the same sequence in every block).
// Two levels: blocks arrive at the counter of their group (blockIdx % 8);
// the last of a group arrives at the global counter; the last overall
// publishes `bar` to the eight group release words, which the blocks poll.
// Split in two so that the next phase's loads are issued between the
// arrival (thread 0, before any of its wave's loads are in flight) and the
// wait.  Callers complete their stores first (stores_done).
__device__ __forceinline__ void barrier_arrive(const StepArgs &A, unsigned bar)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned *sy = A.sync;
        K2_TRACE(2 * bar);
        if (!sync_load(sy + SYNC_ABORT)) {
            const unsigned nb = gridDim.x;
            const unsigned ng = nb < STEP_GROUPS ? nb : STEP_GROUPS;
            const unsigned grp = blockIdx.x % ng;
            const unsigned n_in = (nb - grp + ng - 1) / ng;
            const unsigned old = sync_add(sy + SYNC_GRP + grp * SYNC_STRIDE);
            if (old == bar * n_in - 1) {
                const unsigned old2 = sync_add(sy + SYNC_GLOB);
                if (old2 == bar * ng - 1) {
                    for (unsigned q = 0; q < ng; ++q) sync_store(sy + SYNC_GEN + q * SYNC_STRIDE, bar);
                }
            }
        }
    }
}

// Returns true when the launch is aborting (every block then leaves).
__device__ __forceinline__ bool barrier_wait(const StepArgs &A, unsigned bar, int *flag_lds)
{
    if (threadIdx.x == 0) {
        unsigned *sy = A.sync;
        const unsigned nb = gridDim.x;
        const unsigned ng = nb < STEP_GROUPS ? nb : STEP_GROUPS;
        const unsigned grp = blockIdx.x % ng;
        int abort = sync_load(sy + SYNC_ABORT) != 0;
        int it = 0;
        while (!abort && sync_load(sy + SYNC_GEN + grp * SYNC_STRIDE) < bar) {
            __builtin_amdgcn_s_sleep(2);
            if (++it > STEP_SPIN_LIMIT || sync_load(sy + SYNC_ABORT)) {
                sync_store(sy + SYNC_ABORT, 1u);
                if (A.d_err) coh_store_i(A.d_err, K2_EHIP);
                abort = 1;
            }
        }
        K2_TRACE(2 * bar + 1);
        *flag_lds = abort;
    }
    __syncthreads();
    return *flag_lds != 0;
}

__device__ __forceinline__ bool grid_barrier(const StepArgs &A, unsigned bar, int *flag_lds)
{
    barrier_arrive(A, bar);
    return barrier_wait(A, bar, flag_lds);
}

// this thread's memory operations (its stores in particular) have completed
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0); }

// Stage x [K] (written by other blocks of this grid) into xs in the GEMV's
// permuted layout; with NORM, times GroupedRMSNorm scale and gamma: G equal
// contiguous groups, each divided by sqrt(mean of squares + eps).
template <int EPC, bool NORM>
__device__ __forceinline__ void step_stage_x(float *xs, int S, const float *x, int K,
                                             const float *gamma, int groups, float eps)
{
    __shared__ float red[K2_WAVES_PER_BLOCK][K2_MAX_GROUPS];
    __shared__ float rs[K2_MAX_GROUPS];
    const int gs = K / groups;
    float ss[K2_MAX_GROUPS];
#pragma unroll
    for (int q = 0; q < K2_MAX_GROUPS; ++q) ss[q] = 0.f;
#pragma unroll 4
    for (int i = threadIdx.x * 4; i < K; i += K2_BLOCK * 4) {
        const float4 t = *reinterpret_cast<const float4 *>(x + i);
        *reinterpret_cast<float4 *>(xs + xs_offset<EPC>(i, S)) = t;
        if constexpr (NORM) {
            const float q2 = t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
            const int g = i / gs;
#pragma unroll
            for (int q = 0; q < K2_MAX_GROUPS; ++q) ss[q] += (q == g) ? q2 : 0.f;
        }
    }
    if constexpr (NORM) {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int g = 0; g < K2_MAX_GROUPS; ++g) {
            if (g < groups) {
                const float t = wave_sum(ss[g]);
                if (lane == 0) red[wave][g] = t;
            }
        }
        __syncthreads();
        if (threadIdx.x < groups) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < K2_WAVES_PER_BLOCK; ++w) t += red[w][threadIdx.x];
            rs[threadIdx.x] = 1.0f / sqrtf(t / (float)gs + eps);
        }
        __syncthreads();
        for (int i = threadIdx.x * 4; i < K; i += K2_BLOCK * 4) {
            float4 *p = reinterpret_cast<float4 *>(xs + xs_offset<EPC>(i, S));
            const float r = rs[i / gs];
            const float4 gm = *reinterpret_cast<const float4 *>(gamma + i);
            float4 t = *p;
            t.x = t.x * r * gm.x; t.y = t.y * r * gm.y;
            t.z = t.z * r * gm.z; t.w = t.w * r * gm.w;
            *p = t;
        }
    }
    __syncthreads();
}

template <int WDT, int R, int U, int PRO, int EPI>
__device__ __forceinline__ void step_gemv(const GemvArgs &a, float *xs, int64_t unit, int64_t stride,
                                          int64_t (&rows)[R], bool (&ok)[R], k2_u4 (&w)[U][R],
                                          float (&sc)[U][R], float &best_v, int &best_i,
                                          unsigned bar = 0)
{
    constexpr int EPC = WT<WDT>::EPC;
    const int S = xs_plane(a.K / EPC);
    step_stage_x<EPC, PRO == PRO_NORM>(xs, S, a.x, a.K, a.gamma, a.groups, a.eps);
    if (threadIdx.x == 0) K2_TRACE(1024 + 2 * bar);
    gemv_units<WDT, R, U, 1, EPI, true>(a, xs, S, unit, stride, rows, ok, w, sc, best_v, best_i);
    if (threadIdx.x == 0) K2_TRACE(1024 + 2 * bar + 1);
}

// Phase boundary: this thread's stores complete, the block arrives at the
// barrier, the next phase's first loads are issued, then the block waits
// for the release.  Leaves the kernel when the launch aborts.
#define K2_BOUNDARY(call)                                   \
    do {                                                    \
        stores_done();                                      \
        barrier_arrive(A, ++bar);                           \
        call;                                               \
        if (barrier_wait(A, bar, &flag)) return;            \
    } while (0)

template <int WDT, int KVDT, int HD, int REP>
__global__ __launch_bounds__(K2_BLOCK) __attribute__((amdgpu_waves_per_eu(2, 8)))
void step_kernel(const StepArgs A)
{
    using TL = StepTiles<WDT>;
    extern __shared__ float4 lds4[];
    float *smem = reinterpret_cast<float *>(lds4);
    __shared__ int flag;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = gridDim.x;
    const int64_t unit0 = (int64_t)blockIdx.x * K2_WAVES_PER_BLOCK + wave;
    const int64_t stride = (int64_t)nb * K2_WAVES_PER_BLOCK;
    const int H = A.H, qd = A.n_qh * HD, qkv_rows = (A.n_qh + 2 * A.n_kv) * HD;
    unsigned bar = 0;
    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;

    // weight registers of each phase kind
    int64_t rq[TL::RQ]; bool oq[TL::RQ]; k2_u4 wq[TL::UQ][TL::RQ]; float sq[TL::UQ][TL::RQ];
    int64_t ro[TL::RO]; bool oo[TL::RO]; k2_u4 wo[TL::UO][TL::RO]; float so[TL::UO][TL::RO];
    int64_t rg[TL::RG]; bool og[TL::RG]; k2_u4 wg[TL::UG][TL::RG]; float sg[TL::UG][TL::RG];
    int64_t rd[TL::RD]; bool od[TL::RD]; k2_u4 wd[TL::UD][TL::RD]; float sd[TL::UD][TL::RD];

    // the activation trail: h0, then one slice per layer
    float *const h0 = A.trail;
    auto slice = [&](int l) { return A.trail + ((H + 63) & ~63) + (int64_t)l * A.layer_floats; };
    auto h_in = [&](int l) { return l == 0 ? h0 : slice(l - 1) + A.off_hb; };

    auto qkv_args = [&](int l) {
        const k2_layer &L = A.layers[l];
        GemvArgs g{};
        g.W = L.qkv; g.Sf = (const float *)L.qkv_s; g.S8 = (const uint8_t *)L.qkv_s;
        g.x = h_in(l); g.gamma = L.g_in; g.eps = A.eps; g.groups = A.groups;
        g.y = slice(l) + A.off_qkv;
        g.N = qkv_rows; g.K = H; g.B = 1;
        g.n_units = (qkv_rows + TL::RQ - 1) / TL::RQ;
        return g;
    };
    auto o_args = [&](int l) {
        const k2_layer &L = A.layers[l];
        GemvArgs g{};
        g.W = L.o; g.Sf = (const float *)L.o_s; g.S8 = (const uint8_t *)L.o_s;
        g.x = slice(l) + A.off_o; g.residual = h_in(l); g.y = slice(l) + A.off_ha;
        g.N = H; g.K = qd; g.B = 1;
        g.n_units = (H + TL::RO - 1) / TL::RO;
        return g;
    };
    auto gu_args = [&](int l) {
        const k2_layer &L = A.layers[l];
        GemvArgs g{};
        g.W = L.gu; g.Sf = (const float *)L.gu_s; g.S8 = (const uint8_t *)L.gu_s;
        g.x = slice(l) + A.off_ha; g.gamma = L.g_post; g.eps = A.eps; g.groups = A.groups;
        g.y = slice(l) + A.off_act;
        g.N = 2 * A.inter; g.n_out = A.inter; g.K = H; g.B = 1;
        g.n_units = (A.inter + TL::RG / 2 - 1) / (TL::RG / 2);
        return g;
    };
    auto down_args = [&](int l) {
        const k2_layer &L = A.layers[l];
        GemvArgs g{};
        g.W = L.down; g.Sf = (const float *)L.down_s; g.S8 = (const uint8_t *)L.down_s;
        g.x = slice(l) + A.off_act; g.residual = slice(l) + A.off_ha; g.y = slice(l) + A.off_hb;
        g.N = H; g.K = A.inter; g.B = 1;
        g.n_units = (H + TL::RD - 1) / TL::RD;
        return g;
    };

    // ---- embedding: h0 = E[token] ------------------------------------------
    {
        int token = A.d_token ? *A.d_token : A.token;
        if (token < 0 || token >= A.vocab) {
            if (blockIdx.x == 0 && tid == 0 && A.d_err) coh_store_i(A.d_err, K2_ERANGE);
            token = 0;
        }
        for (int i = blockIdx.x * K2_BLOCK + tid; i < H; i += nb * K2_BLOCK) {
            float v;
            if (A.embdt == K2_BF16)
                v = bf16_to_f32(reinterpret_cast<const uint16_t *>(A.embed)[(int64_t)token * H + i]);
            else
                v = reinterpret_cast<const float *>(A.embed)[(int64_t)token * H + i];
            coh_store(h0 + i, v);
        }
    }
    K2_BOUNDARY((gemv_prefetch<WDT, TL::RQ, TL::UQ, EPI_PLAIN>(qkv_args(0), unit0, rq, oq, wq, sq)));

    AttnArgs at{};
    at.cos_sin = A.rope; at.part = A.part; at.part_ml = A.part_ml;
    at.n_qh = A.n_qh; at.n_kv = A.n_kv; at.cap = A.cap; at.len = A.len; at.pos = A.pos;
    at.chunk = A.attn_chunk; at.S = A.attn_S; at.scale = A.scale;
    const int n_items = A.n_kv * A.attn_S;

    // layer 0's QKV, then per layer: attention, O, gate/up, down and (but
    // for the last layer) the next layer's QKV, so that every prefetch is
    // consumed in the iteration that issued it
    step_gemv<WDT, TL::RQ, TL::UQ, PRO_NORM, EPI_PLAIN>(qkv_args(0), smem, unit0, stride, rq, oq, wq,
                                                        sq, best_v, best_i, bar);
#pragma unroll 1
    for (int l = 0;; ++l) {
        const k2_layer &L = A.layers[l];
        stores_done();
        if (grid_barrier(A, ++bar, &flag)) return;
        // ---- RoPE + KV append + attention (+ combine by the last split) --------
        at.qkv = slice(l) + A.off_qkv;
        at.out = slice(l) + A.off_o;
        at.kc = L.kc; at.vc = L.vc; at.ks = L.ks; at.vs = L.vs;
        for (int item = blockIdx.x; item < n_items; item += nb) {
            const int g = item % A.n_kv, s = item / A.n_kv;
            attn_block<KVDT, HD, REP, true, K2_WAVES_PER_BLOCK, true, true>(at, g, s, A.attn_S, smem);
            if (A.attn_S > 1) {
                stores_done();                     // partial stores complete
                __syncthreads();
                if (tid == 0) {
                    unsigned *c = A.sync + SYNC_HEAD + g * SYNC_STRIDE;
                    const unsigned old = sync_add(c);
                    flag = old == (unsigned)A.attn_S - 1;
                    if (flag) sync_store(c, 0u);   // reused by the next layer
                }
                __syncthreads();
                if (flag) attn_combine_block<HD, REP, true>(at, g, smem);
                __syncthreads();
            }
        }
        K2_BOUNDARY((gemv_prefetch<WDT, TL::RO, TL::UO, EPI_PLAIN>(o_args(l), unit0, ro, oo, wo, so)));
        // ---- O + residual ------------------------------------------------------
        step_gemv<WDT, TL::RO, TL::UO, PRO_NONE, EPI_PLAIN>(o_args(l), smem, unit0, stride, ro, oo, wo,
                                                            so, best_v, best_i, bar);
        K2_BOUNDARY((gemv_prefetch<WDT, TL::RG, TL::UG, EPI_SWIGLU>(gu_args(l), unit0, rg, og, wg, sg)));
        // ---- gate/up + SwiGLU --------------------------------------------------
        step_gemv<WDT, TL::RG, TL::UG, PRO_NORM, EPI_SWIGLU>(gu_args(l), smem, unit0, stride, rg, og,
                                                             wg, sg, best_v, best_i, bar);
        K2_BOUNDARY((gemv_prefetch<WDT, TL::RD, TL::UD, EPI_PLAIN>(down_args(l), unit0, rd, od, wd, sd)));
        // ---- down + residual ---------------------------------------------------
        step_gemv<WDT, TL::RD, TL::UD, PRO_NONE, EPI_PLAIN>(down_args(l), smem, unit0, stride, rd, od,
                                                            wd, sd, best_v, best_i, bar);
        if (l + 1 == A.n_layers) break;
        // ---- next layer's QKV --------------------------------------------------
        K2_BOUNDARY((gemv_prefetch<WDT, TL::RQ, TL::UQ, EPI_PLAIN>(qkv_args(l + 1), unit0, rq, oq, wq, sq)));
        step_gemv<WDT, TL::RQ, TL::UQ, PRO_NORM, EPI_PLAIN>(qkv_args(l + 1), smem, unit0, stride, rq, oq,
                                                            wq, sq, best_v, best_i, bar);
    }

    // ---- final norm + lm_head + argmax -------------------------------------------
    if (!A.logits) return;
    {
        GemvArgs g{};
        g.W = A.lm; g.Sf = (const float *)A.lm_s; g.S8 = (const uint8_t *)A.lm_s;
        g.x = h_in(A.n_layers); g.gamma = A.g_final; g.eps = A.eps; g.groups = A.groups;
        g.y = A.logits;
        g.N = A.vocab; g.K = H; g.B = 1;
        g.n_units = (A.vocab + TL::RL - 1) / TL::RL;
        int64_t rl[TL::RL]; bool ol[TL::RL]; k2_u4 wl[TL::UL][TL::RL]; float sl[TL::UL][TL::RL];
        K2_BOUNDARY((gemv_prefetch<WDT, TL::RL, TL::UL, EPI_ARGMAX>(g, unit0, rl, ol, wl, sl)));
        step_gemv<WDT, TL::RL, TL::UL, PRO_NORM, EPI_ARGMAX>(g, smem, unit0, stride, rl, ol, wl, sl,
                                                             best_v, best_i, bar);
    }
    argmax_block(best_v, best_i);
    if (tid == 0) {
        coh_store(A.am_v + blockIdx.x, best_v);
        coh_store_i(A.am_i + blockIdx.x, best_i);
        stores_done();
        flag = sync_add(A.sync + SYNC_AM) == (unsigned)nb - 1;
    }
    __syncthreads();
    if (!flag) return;
    // the last block: reduce the candidates in block order (fixed order)
    float v = -INFINITY;
    int i = 0x7FFFFFFF;
    for (int b = tid; b < nb; b += K2_BLOCK) argmax_pair_max(v, i, coh_load(A.am_v + b), coh_load_i(A.am_i + b));
    argmax_block(v, i);
    if (tid == 0 && A.next) *A.next = i;
}

#undef K2_BOUNDARY

// ------------------------------------------------------------------ host --

template <int WDT, int KVDT, int HD, int REP>
constexpr size_t step_lds_bytes_t(int H, int qd, int inter)
{
    constexpr int EPC = WT<WDT>::EPC;
    size_t f = 0;
    for (int K : {H, qd, inter}) {
        const size_t x = (size_t)EPC * xs_plane(K / EPC);
        f = x > f ? x : f;
    }
    const size_t at = attn_lds_floats<HD, REP, K2_WAVES_PER_BLOCK>();
    const size_t cb = combine_lds_floats<REP>();
    f = at > f ? at : f;
    f = cb > f ? cb : f;
    return f * sizeof(float);
}

// Cooperative launch of the step kernel on as many blocks as can be
// resident together (at most max_blocks).
template <int WDT, int KVDT, int HD, int REP>
int step_launch_t(const StepArgs &A, int H, int qd, int inter, int max_blocks, hipStream_t st)
{
    auto kern = step_kernel<WDT, KVDT, HD, REP>;
    const size_t lds = step_lds_bytes_t<WDT, KVDT, HD, REP>(H, qd, inter);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return K2_EHIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return K2_EHIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, K2_BLOCK, lds) != hipSuccess)
        return K2_EHIP;
    if (per_cu < 1 || cus < 1) return K2_EUNSUPPORTED;
    int nb = cus * per_cu;
    if (nb > max_blocks) nb = max_blocks;
    StepArgs a = A;
    void *args[] = {(void *)&a};
    if (hipLaunchCooperativeKernel((const void *)kern, dim3(nb), dim3(K2_BLOCK), args, (unsigned)lds,
                                   st) != hipSuccess)
        return K2_EHIP;
    return K2_OK;
}

template <int WDT>
int step_dispatch_t(int kvdt, int hd, int rep, const StepArgs &A, int H, int qd, int inter,
                    int max_blocks, hipStream_t st)
{
#define K2_STEP(KV, HDV, RP)                                                                        \
    if (kvdt == KV && hd == HDV && rep == RP)                                                      \
        return step_launch_t<WDT, KV, HDV, RP>(A, H, qd, inter, max_blocks, st);
#define K2_STEP_KV(KV) K2_STEP(KV, 128, 4) K2_STEP(KV, 128, 2) K2_STEP(KV, 16, 2) K2_STEP(KV, 16, 4)
    K2_STEP_KV(K2_F32)
    K2_STEP_KV(K2_BF16)
    K2_STEP_KV(K2_I8)
#undef K2_STEP_KV
#undef K2_STEP
    return K2_EUNSUPPORTED;
}

}  // namespace k2
