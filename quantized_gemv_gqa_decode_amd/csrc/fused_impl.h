// fused_impl.h -- QKV projection, attention and O projection of one layer as
// ONE launch whose blocks wait only for the blocks whose output they read.
//
// Kernel-per-phase, every phase pays a launch-to-launch gap and then the
// latency of its first weight bytes (together ~3 us, more than the O
// projection streams).  Here one grid holds, in block order:
//   [QKV GEMV blocks | attention blocks (split x kv head) | O GEMV blocks]
// and dependencies are counters in a per-layer sync area that the host
// clears once per position:
//   * a QKV block stores its rows at device scope, waits for the stores,
//     and adds its row count to the counter of their kv head;
//   * an attention block first issues the copies of its K/V tiles (they do
//     not depend on this launch), then waits until its kv head has all of
//     its (REP + 2) * head_dim rows, then reads q, k, v at device scope;
//     the block that completes a kv head (the combiner, or the only split)
//     stores the head's output, waits for it and bumps the heads counter;
//   * an O block first loads its weights into registers, then waits until
//     every kv head is complete, then stages the attention output (device
//     scope) and finishes like the stand-alone GEMV.
// Every block waits only for blocks with lower indices.  Blocks start in
// index order, so the lowest unfinished block always runs and everything it
// waits for has finished: the grid cannot deadlock, whatever fits on the
// chip at once.  Every wait is bounded (block_wait_count) and reports
// K2_EHIP through d_err instead of hanging.
//
// One launch has one block size and one LDS size: all roles use 256 threads,
// and the attention role uses the lean stream shape (4 waves, 2 stages of
// 8 KiB tiles) so that its LDS stays close to the GEMVs' staged activations.
#pragma once
#include "attn_impl.h"
#include "gemv_impl.h"

namespace k2 {

using StreamLean = StreamCfg<4, 2, 8192>;

// per-layer sync words (unsigned), zeroed once per position.  A QKV block
// sets its own flag (a plain device-scope store: hundreds of blocks adding
// into a few counters would serialize on one cache line); the kv-head
// completions are counted, and the last one raises a ready flag that is
// replicated on separate 256-byte lines so that the O blocks' polling is
// spread over several memory channels.
constexpr int FUSE_MAX_QKV_BLOCKS = 2048;
constexpr int FUSE_SYNC_FLAGS = 0;                          // [QKV block] done
constexpr int FUSE_SYNC_HEADS = FUSE_MAX_QKV_BLOCKS;        // kv heads complete (counter)
constexpr int FUSE_READY_COPIES = 16;
constexpr int FUSE_SYNC_READY = FUSE_SYNC_HEADS + 64;       // [copy * 64]: all heads complete
constexpr int FUSE_SYNC_WORDS = FUSE_SYNC_READY + FUSE_READY_COPIES * 64;
constexpr int FUSE_MAX_KV = 64;

// GEMV tiles (rows per wave unit, 16-byte chunks per lane per pass) of the
// QKV and O roles per weight format: the stand-alone tile choice for the
// 3.7B shape (QKV 6144 x 2560, O 2560 x 4096).  RQ = 2 makes a QKV block 8
// rows, so a block never straddles two kv heads of head_dim 128.
template <int WDT> struct FusedTiles;
template <> struct FusedTiles<K2_F32>     { static constexpr int RQ = 2, UQ = 10, RO = 1, UO = 10; };
template <> struct FusedTiles<K2_BF16>    { static constexpr int RQ = 2, UQ = 5, RO = 1, UO = 10; };
template <> struct FusedTiles<K2_FP8E4M3> { static constexpr int RQ = 2, UQ = 3, RO = 1, UO = 5; };
template <> struct FusedTiles<K2_MXFP4>   { static constexpr int RQ = 2, UQ = 2, RO = 1, UO = 2; };

struct FusedArgs {
    GemvArgs q;            // QKV: x = h (norm prologue), y = qkv (device-scope stores)
    GemvArgs o;            // O: x = attention output, y = residual = h
    AttnArgs at;           // fused RoPE + append + attention, qkv = q.y, out = o.x
    unsigned *sync;        // this layer's FUSE_SYNC_WORDS words
    int32_t *d_err;        // nullable
    int nq, na;            // QKV blocks, attention blocks (O blocks follow)
};

// kv head of q/k/v row r
template <int HD, int REP>
__device__ __forceinline__ int fused_row_head(int r, int n_qh, int n_kv)
{
    if (r < n_qh * HD) return r / (REP * HD);
    r -= n_qh * HD;
    return (r < n_kv * HD ? r : r - n_kv * HD) / HD;
}

template <int WDT, int HD, int REP, int XV>
__device__ __forceinline__ void fused_qkv_role(const FusedArgs &f, int blk, float *xs)
{
    using TL = FusedTiles<WDT>;
    constexpr int R = TL::RQ, U = TL::UQ, EPC = WT<WDT>::EPC;
    const GemvArgs &a = f.q;
    const int S = xs_plane(a.K / EPC);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t unit = (int64_t)blk * K2_WAVES_PER_BLOCK + wave;
    const int64_t stride = (int64_t)f.nq * K2_WAVES_PER_BLOCK;
    float best_v = 0.f;
    int best_i = 0;
    int64_t rows[R];
    bool ok[R];
    k2_u4 w[U][R];
    float sc[U][R];
    float4 xr[XV];
    issue_x<XV>(a, xr);
    gemv_prefetch<WDT, R, U, EPI_PLAIN>(a, unit, rows, ok, w, sc);
    finish_x<XV, PRO_NORM, EPC>(xs, a, xr, S);
    K2_ATRACE(5);
    gemv_units<WDT, R, U, 1, EPI_PLAIN, true>(a, xs, S, unit, stride, rows, ok, w, sc, best_v, best_i);
    K2_ATRACE(6);
    // this block's rows are stored: raise its flag
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(f.sync + FUSE_SYNC_FLAGS + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every QKV block holding rows of kv head g has raised its flag
// (wave 0 polls: q rows, then k rows, then v rows of the head; RB rows per
// block).  Bounded like block_wait_count.
template <int HD, int REP, int RB>
__device__ __forceinline__ void fused_wait_head(const FusedArgs &f, int g)
{
    static_assert(HD % RB == 0, "a QKV block never straddles two kv heads");
    constexpr int NQB = REP * HD / RB, NKB = HD / RB, NB = NQB + 2 * NKB;
    const unsigned *fl = f.sync + FUSE_SYNC_FLAGS;
    const int qb0 = g * NQB, kb0 = (f.at.n_qh * HD + g * HD) / RB, vb0 = kb0 + f.at.n_kv * HD / RB;
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < K2_WAVE) {
        int spins = 0;
        bool all;
        do {
            bool mine = true;
            for (int j = lane; j < NB; j += K2_WAVE) {
                const int b = j < NQB ? qb0 + j : j < NQB + NKB ? kb0 + (j - NQB) : vb0 + (j - NQB - NKB);
                mine &= coh_load_u(fl + b) != 0u;
            }
            all = __all(mine);
            if (!all) __builtin_amdgcn_s_sleep(K2_WAIT_SLEEP);
        } while (!all && ++spins < K2_WAIT_SPIN_LIMIT);
        if (!all && lane == 0 && f.d_err) coh_store_i(f.d_err, K2_EHIP);
    }
    __syncthreads();
}

template <int WDT, int KVDT, int HD, int REP>
__device__ __forceinline__ void fused_attn_role(const FusedArgs &f, int ab, float *smem)
{
    const AttnArgs &a = f.at;
    const int S = a.S, s = ab % S, g = ab / S;
    uint32_t kv_bits = 0u;
    float kv_scale = 0.f;
    const bool holder = attn_stream_block<KVDT, HD, REP, true, true, StreamLean, true>(
        a, g, s, S, smem, kv_bits, kv_scale, [&] { fused_wait_head<HD, REP, 4 * FusedTiles<WDT>::RQ>(f, g); });
    __shared__ int complete;                       // this block finished kv head g
    if (S > 1) {
        __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores completed
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(a.head_cnt + g, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            complete = old == (unsigned)S - 1;
            if (complete) __hip_atomic_store(a.head_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (complete) attn_combine_block<HD, REP, true, K2_BLOCK>(a, g, smem);
    } else {
        if (threadIdx.x == 0) complete = 1;
        __syncthreads();
    }
    if (complete) {                                // the head's output is out: count it
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned done = __hip_atomic_fetch_add(f.sync + FUSE_SYNC_HEADS, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            if (done == (unsigned)a.n_kv - 1)          // the last head: raise every ready copy
                for (int c = 0; c < FUSE_READY_COPIES; ++c)
                    __hip_atomic_store(f.sync + FUSE_SYNC_READY + c * 64, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the new position's K/V: no block of this launch reads slot pos
    if (holder) kv_write_head<KVDT, HD>(kv_bits, kv_scale, a.kc, a.vc, a.ks, a.vs, g, a.cap, a.pos);
}

template <int WDT, int XV>
__device__ __forceinline__ void fused_o_role(const FusedArgs &f, int ob, float *xs)
{
    using TL = FusedTiles<WDT>;
    constexpr int R = TL::RO, U = TL::UO, EPC = WT<WDT>::EPC;
    const GemvArgs &a = f.o;
    const int S = xs_plane(a.K / EPC);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nob = gridDim.x - f.nq - f.na;
    const int64_t unit = (int64_t)ob * K2_WAVES_PER_BLOCK + wave;
    const int64_t stride = (int64_t)nob * K2_WAVES_PER_BLOCK;
    float best_v = 0.f;
    int best_i = 0;
    int64_t rows[R];
    bool ok[R];
    k2_u4 w[U][R];
    float sc[U][R];
    gemv_prefetch<WDT, R, U, EPI_PLAIN>(a, unit, rows, ok, w, sc);   // weights before the wait
    block_wait_count(f.sync + FUSE_SYNC_READY + (ob % FUSE_READY_COPIES) * 64, 1u, f.d_err);
    K2_ATRACE(5);
    float4 xr[XV];
    issue_x<XV, true>(a, xr);                      // the attention output, device scope
    finish_x<XV, PRO_NONE, EPC>(xs, a, xr, S);
    K2_ATRACE(6);
    gemv_units<WDT, R, U, 1, EPI_PLAIN, false>(a, xs, S, unit, stride, rows, ok, w, sc, best_v, best_i);
}

template <int WDT, int KVDT, int HD, int REP, int XVQ, int XVO>
__global__ __launch_bounds__(K2_BLOCK) void fused_qao_kernel(const FusedArgs f)
{
    extern __shared__ float4 lds4[];
    float *smem = reinterpret_cast<float *>(lds4);
    const int b = blockIdx.x;
    K2_ATRACE_CLEAR();
    K2_ATRACE(0);
    if (b < f.nq) fused_qkv_role<WDT, HD, REP, XVQ>(f, b, smem);
    else if (b < f.nq + f.na) fused_attn_role<WDT, KVDT, HD, REP>(f, b - f.nq, smem);
    else fused_o_role<WDT, XVO>(f, b - f.nq - f.na, smem);
    K2_ATRACE(11);
    K2_ATRACE_FLUSH();
}

// ------------------------------------------------ attention + O, one launch --
//
// Grid (1-D), in block order: [attention blocks (split s, kv head g) | O
// GEMV blocks].  Both roles use the stand-alone attention block shape
// (ATT_NT threads, its LDS ring), so the attention role is exactly the
// stand-alone kernel's.  An O block first issues the loads of ALL of its
// weight rows (R rows per wave, U chunks per lane: one pass of the whole
// row), then waits for the ready flag, stages the attention output (device
// scope) and finishes like the stand-alone GEMV: its weights were streaming
// while the attention ran.
//   * the block that completes kv head g (its combiner, or the only split)
//     stores the head's output at device scope, waits for the stores and
//     counts the head; the last head raises every ready copy;
//   * every O block counts itself when done; the last one clears the
//     counters and flags, so the sync words are zero between launches.
// Blocks start in index order and an O block waits only for attention
// blocks (lower indices), so the grid cannot deadlock whatever fits on the
// chip; the host launches this form only when everything fits at once, so
// the O weights really stream during the attention.  The wait is bounded
// (block_wait_count) and reports K2_EHIP through d_err instead of hanging.
// The O rows are summed in the same order as by the stand-alone GEMV with
// one pass per row, so the result is bit-identical to attention + GEMV.

struct AttnOArgs {
    AttnArgs at;           // RoPE + append + attention (fused form), out = o.x
    GemvArgs o;            // O: x = attention output, y = residual = h
    int32_t *d_err;        // nullable
    int na;                // attention blocks (S * n_kv); O blocks follow
};

// An O block holds its weight loads back this long (100 MHz ticks): issued
// at once, the O rows' bytes sit in the memory queues ahead of the
// attention's first cache tiles and delay its whole dependent chain.  1.2 us
// lets those go first and still lands the O rows well before the attention
// ends (3.7B shape: ~2 % faster per decode step than no hold-back).
constexpr int AO_O_DELAY_TICKS = 120;

template <int KVDT, int HD, int REP>
__device__ __forceinline__ void ao_attn_role(const AttnOArgs &f, int ab, float *smem)
{
    const AttnArgs &a = f.at;
    const int S = a.S, s = ab % S, g = ab / S;
    unsigned *sync = a.ao_sync;
    uint32_t kv_bits = 0u;
    float kv_scale = 0.f;
    const bool holder = attn_stream_block<KVDT, HD, REP, true, true>(a, g, s, S, smem, kv_bits, kv_scale);
    __shared__ int complete;                       // this block finished kv head g
    if (S > 1) {
        __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores completed
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(a.head_cnt + g, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            complete = old == (unsigned)S - 1;
            if (complete) __hip_atomic_store(a.head_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (complete) attn_combine_block<HD, REP, true, ATT_NT>(a, g, smem);
    } else {
        if (threadIdx.x == 0) complete = 1;
        __syncthreads();
    }
    if (complete) {                                // the head's output is stored: count it
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned done = __hip_atomic_fetch_add(sync + AO_SYNC_HEADS, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            if (done == (unsigned)a.n_kv - 1)
                for (int c = 0; c < AO_READY_COPIES; ++c)
                    __hip_atomic_store(sync + AO_SYNC_READY + c * 64, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the new position's K/V: no block of this launch reads slot pos
    if (holder) kv_write_head<KVDT, HD>(kv_bits, kv_scale, a.kc, a.vc, a.ks, a.vs, g, a.cap, a.pos);
}

template <int WDT, int R, int U>
__device__ __forceinline__ void ao_o_role(const AttnOArgs &f, int ob, float *xs)
{
    constexpr int EPC = WT<WDT>::EPC, WPB = ATT_NT / K2_WAVE;
    const GemvArgs &a = f.o;
    unsigned *sync = f.at.ao_sync;
    const int S = xs_plane(a.K / EPC);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nob = (int)gridDim.x - f.na;
    const int64_t unit = (int64_t)ob * WPB + wave;
    const int64_t stride = (int64_t)nob * WPB;
    float best_v = 0.f;
    int best_i = 0;
    int64_t rows[R];
    bool ok[R];
    k2_u4 w[U][R];
    float sc[U][R];
    {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)AO_O_DELAY_TICKS) __builtin_amdgcn_s_sleep(2);
    }
    gemv_prefetch<WDT, R, U, EPI_PLAIN>(a, unit, rows, ok, w, sc);   // weights before the wait
    block_wait_count(sync + AO_SYNC_READY + (ob % AO_READY_COPIES) * 64, 1u, f.d_err);
    // the attention output (B = 1), device scope, into the GEMV's LDS planes
    for (int i = threadIdx.x * 4; i < a.K; i += ATT_NT * 4)
        *reinterpret_cast<float4 *>(xs + xs_offset<EPC>(i, S)) = ld4<true>(a.x, i);
    __syncthreads();
    gemv_units<WDT, R, U, 1, EPI_PLAIN, false>(a, xs, S, unit, stride, rows, ok, w, sc, best_v, best_i);
    __syncthreads();                               // every wave of the block is past its wait
    if (threadIdx.x == 0) {
        const unsigned d = __hip_atomic_fetch_add(sync + AO_SYNC_ODONE, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        if (d == (unsigned)nob - 1) {              // the last O block: clear for the next launch
            __hip_atomic_store(sync + AO_SYNC_HEADS, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int c = 0; c < AO_READY_COPIES; ++c)
                __hip_atomic_store(sync + AO_SYNC_READY + c * 64, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + AO_SYNC_ODONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int WDT, int KVDT, int HD, int REP, int R, int U>
__global__ __launch_bounds__(ATT_NT) void attn_o_kernel(const AttnOArgs f)
{
    extern __shared__ float4 lds4[];
    float *smem = reinterpret_cast<float *>(lds4);
    const int b = blockIdx.x;
    if (b < f.na) ao_attn_role<KVDT, HD, REP>(f, b, smem);
    else ao_o_role<WDT, R, U>(f, b - f.na, smem);
}

}  // namespace k2
