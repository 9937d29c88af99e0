// attn_o_impl.h -- attention of one decode position and the O projection
// (+ residual) as ONE launch ([k2-burn] "Project layout": layer.rs, the
// attention residual).
//
// Kernel-per-phase, the O projection would pay a launch-to-launch gap and
// then the latency of its first weight bytes (together ~3 us, about what
// its 21 MB stream at the 3.7B shape takes).  Here its blocks are resident
// beside the attention blocks and load their weight rows while the
// attention runs.
#pragma once
#include "attn_impl.h"
#include "gemv_impl.h"

namespace k2 {

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
//     counts the head; the last head raises every copy of the ready word
//     (one per 256-byte line), and an O block polls its copy.  Measured
//     against one flag per head that every O block polls for all heads:
//     2.139 against 2.219 ms per decode step (3.7B shape, same build and
//     box), the fewer polled words winning;
//   * every O block counts itself when done; the last one clears the
//     counters and flags, so the sync words are zero between launches.
// Blocks start in index order and an O block waits only for attention
// blocks (lower indices), so the grid cannot deadlock whatever fits on the
// chip; the host launches this form only when both roles fit at once, so
// the O weights really stream during the attention.  With a device
// position (AttnArgs::d_pos) the attention part of the grid has the split
// extent that fits beside the O blocks: the blocks past the device split
// count leave at once, and where the position needs more splits than that
// each block takes a longer range (attn_resolve_pos); on a position outside
// the cache every block leaves at once and nothing is written.  The wait is bounded
// (block_wait_count) and reports K2_EHIP through d_err instead of hanging.
// The O rows are summed in the same order as by the stand-alone GEMV with
// one pass per row, so the result is bit-identical to attention + GEMV.

struct AttnOArgs {
    AttnArgs at;           // RoPE + append + attention (fused form), out = o.x
    GemvArgs o;            // O: x = attention output, y = residual = h
    int32_t *d_err;        // nullable
    int na;                // attention blocks (grid split extent * n_kv); O blocks follow
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
    const int Sg = f.na / a.n_kv;                  // the grid's split extent
    const int s = ab % Sg, g = ab / Sg;
    if (s >= a.S) return;                          // device split count below it
    const int S = a.S;
    unsigned *sync = a.ao_sync;
    uint32_t kv_bits = 0u;
    float kv_scale = 0.f;
    const bool holder = attn_stream_block<KVDT, HD, REP, true, true>(a, g, s, S, smem, kv_bits, kv_scale);
    __shared__ int complete;                       // this block finished kv head g
    if (S > 1) {
        __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores completed
        __syncthreads();
        K2_ATRACE(4);
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(a.head_cnt + g, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            complete = old == (unsigned)S - 1;
            if (complete) __hip_atomic_store(a.head_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        K2_ATRACE(5);
        if (complete) {
            attn_combine_block<HD, REP, true, ATT_NT>(a, g, smem);
            K2_ATRACE(6);
        }
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
            if (done == (unsigned)a.n_kv - 1)      // the last head: raise every ready copy
                for (int c = 0; c < AO_READY_COPIES; ++c)
                    __hip_atomic_store(sync + AO_SYNC_READY + c * 64, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the new position's K/V: no block of this launch reads slot pos
    if (holder) kv_write_head<KVDT, HD>(kv_bits, kv_scale, a.kc, a.vc, a.ks, a.vs, g, a.cap, a.pos);
    K2_ATRACE(11);
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
    K2_ATRACE(0);
    {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)AO_O_DELAY_TICKS) __builtin_amdgcn_s_sleep(2);
    }
    K2_ATRACE(1);
    gemv_prefetch<WDT, R, U, EPI_PLAIN>(a, unit, rows, ok, w, sc);   // weights before the wait
    K2_ATRACE(2);
    block_wait_count(sync + AO_SYNC_READY + (ob % AO_READY_COPIES) * 64, 1u, f.d_err);
    K2_ATRACE(3);
    // the attention output (B = 1), device scope, into the GEMV's LDS planes
    for (int i = threadIdx.x * 4; i < a.K; i += ATT_NT * 4)
        *reinterpret_cast<float4 *>(xs + xs_offset<EPC>(i, S)) = ld4<true>(a.x, i);
    __syncthreads();
    K2_ATRACE(4);
    gemv_units<WDT, R, U, 1, EPI_PLAIN, false>(a, xs, S, unit, stride, rows, ok, w, sc, best_v, best_i);
    __syncthreads();                               // every wave of the block is past its wait
    K2_ATRACE(5);
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
    K2_ATRACE(11);
}

template <int WDT, int KVDT, int HD, int REP, int R, int U>
__global__ __launch_bounds__(ATT_NT) void attn_o_kernel(const AttnOArgs f0)
{
    extern __shared__ float4 lds4[];
    float *smem = reinterpret_cast<float *>(lds4);
    AttnOArgs f = f0;
    if (!attn_resolve_pos(f.at, f.na / f.at.n_kv)) return;   // nothing is written
    K2_ATRACE_CLEAR();
    const int b = blockIdx.x;
    if (b < f.na) ao_attn_role<KVDT, HD, REP>(f, b, smem);
    else ao_o_role<WDT, R, U>(f, b - f.na, smem);
    K2_ATRACE_FLUSH();
}

}  // namespace k2
