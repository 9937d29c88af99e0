// attn_impl.h -- device code of the split-K GQA decode attention (included
// by attn.hip for the stand-alone kernels, by attn_rows.hip for a prefill
// chunk's queries and by attn_o_impl.h for the attention + O launch).
//
// Semantics ([k2-burn] "Model shape": GQA with 4x KV repeat; "Limitations":
// plain SDPA, softmax in fp32; "KV cache storage": fp32 / bf16 / symmetric
// int8 with one scale per head_dim block):
//   out[h] = softmax_j(q_h . K_hat[g][j] * scale) V_hat[g][j],  g = h / rep,
// over positions j in [0, len).
//
// Grid: (S splits, n_kv heads); block = ATT_NT threads (8 waves, the
// StreamFor shape below).  Block (s, g) handles positions
// [s*chunk, min(len, (s+1)*chunk)) for the rep query heads of kv head g:
//   1. the rep query heads are rotated (fused form) and scaled into LDS;
//   2. K and V rows stream through a ring of LDS stages filled by LDS-DMA
//      (global_load_lds), the next tiles in flight while one is computed; a row
//      of head_dim values is split over LPP lanes (16 bytes each), so one
//      wave covers 64/LPP positions per slot; the int8 per-position scale
//      multiplies the finished dot product and is folded into the
//      probability for V;
//   3. each wave keeps an online fp32 softmax (running max, rescaled sum and
//      accumulator); the waves are merged through LDS;
//   4. with one split the normalised output is written directly; otherwise
//      every block publishes (max, sum, unnormalised o) at device scope, and
//      the last block of the kv head to finish combines the S partials in
//      split order (fixed order: the result is run-to-run deterministic).
// Fused form: the block holding the new position `pos` also rotates k, stores
// k and v at slot pos in the cache format, and uses the stored (dequantized)
// values for that position from LDS.
#pragma once
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

template <int KVDT> struct KVT;
template <> struct KVT<K2_F32>  { static constexpr int EPC = 4;  using T = float;    };
template <> struct KVT<K2_BF16> { static constexpr int EPC = 8;  using T = uint16_t; };
template <> struct KVT<K2_I8>   { static constexpr int EPC = 16; using T = int8_t;   };

template <int KVDT> __device__ __forceinline__ void kv_decode(const k2_u4 w, float *v);

constexpr float K2_LOG2E = 1.4426950408889634f;
constexpr float K2_LN2 = 0.6931471805599453f;
// Slack of the streaming blocks' lazily moved softmax reference (base 2):
// every weight stays <= 2^8, far from the fp32 range.
constexpr float ATT_SLACK = 8.0f;

// 2^x with the hardware exponential (x <= 0 here; -inf gives 0)
__device__ __forceinline__ float k2_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x plus its value in lane ^ 16 (permlane16_swap) or lane ^ 32
// (permlane32_swap): VALU lane swaps, no LDS; every lane of a pair gets the
// same bits.
__device__ __forceinline__ float xor16_add(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_add(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce-scatter over the position groups of a wave (lanes that share
// lane % LPP, group = lane / LPP, LPP in {8, 16, 32}): each step pairs value
// i with value i + n/2 and one lane swap leaves the sum of the first in the
// lanes whose group bit is 0 and the sum of the second in the others, so
// every step halves the values per lane.  On return v[j], j < NV * LPP / 64,
// holds the total over the groups of value j + (NV * LPP / 64) * group.
template <int NV, int LPP>
__device__ __forceinline__ void group_reduce_scatter(float (&v)[NV], int lane)
{
    static_assert(LPP == 8 || LPP == 16 || LPP == 32, "group bits 3..5");
    static_assert(NV % (64 / LPP) == 0, "values split evenly");
    if constexpr (LPP <= 32) {                     // group bit 5: lane ^ 32
#pragma unroll
        for (int i = 0; i < NV / 2; ++i) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + NV / 2]),
                                                            false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    }
    if constexpr (LPP <= 16) {                     // group bit 4: lane ^ 16 (rows)
        constexpr int n = NV / 2;                  // values left after bit 5
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + n / 2]),
                                                            false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    }
    if constexpr (LPP <= 8) {                      // group bit 3: lane ^ 8 inside a row
        constexpr int n = NV / 4;                  // values left after bits 5 and 4
        const bool hi = (lane & 8) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float keep = hi ? v[i + n / 2] : v[i];
            const float send = hi ? v[i] : v[i + n / 2];
            v[i] = keep + dpp<0x128>(send);        // row_ror:8 reads lane ^ 8
        }
    }
}

// Sum over the lanes that share lane % LPP (the 64 / LPP position groups of
// a wave), result in every lane: rotations inside rows of 16 (row_ror by 8,
// 4, ... down to LPP), then the lane swaps across rows and halves.
template <int LPP>
__device__ __forceinline__ float subgroup_sum(float x)
{
    if constexpr (LPP <= 8) x += dpp<0x128>(x);
    if constexpr (LPP <= 4) x += dpp<0x124>(x);
    if constexpr (LPP <= 2) x += dpp<0x122>(x);
    if constexpr (LPP <= 1) x += dpp<0x121>(x);
    if constexpr (LPP <= 16) x = xor16_add(x);
    if constexpr (LPP <= 32) x = xor32_add(x);
    return x;
}

// decode one 16-byte cache chunk into EPC floats; int8 as unsigned bytes
// u = code + 128 (one convert per element; callers subtract the offset)
template <int KVDT>
__device__ __forceinline__ void kv_decode_u(const k2_u4 w, float *v)
{
    if constexpr (KVDT == K2_I8) {
        const uint32_t ws[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u,
                                w.w ^ 0x80808080u};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) v[4 * i + b] = (float)((ws[i] >> (8 * b)) & 0xFFu);
    } else {
        kv_decode<KVDT>(w, v);
    }
}

// decode one 16-byte cache chunk into EPC floats (int8: the raw codes)
template <int KVDT>
__device__ __forceinline__ void kv_decode(const k2_u4 w, float *v)
{
    if constexpr (KVDT == K2_F32) {
        v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
        v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    } else if constexpr (KVDT == K2_BF16) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(ws[i]); v[2 * i + 1] = bf16_hi(ws[i]); }
    } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) v[4 * i + b] = (float)(int8_t)(ws[i] >> (8 * b));
    }
}

// Block barrier for data exchanged through LDS only: waits for this wave's
// LDS operations, not for its global loads (LDS-DMA copies in flight stay
// in flight, unlike __syncthreads, whose fence waits for them).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0); vmcnt, expcnt not waited
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <bool RAW>
__device__ __forceinline__ void block_sync()
{
    if constexpr (RAW) lds_barrier();
    else __syncthreads();
}

// Largest |x| over the head_dim values of k (threads [0, HD)) and of v
// (threads [HD, 2 HD)); every thread must call it.  RAW: LDS-only barriers.
template <int HD, bool RAW = false>
__device__ __forceinline__ float kv_head_absmax(float ax, float *tmp4)
{
    constexpr int W = HD < 64 ? HD : 64;
    float m = ax;
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, K2_WAVE));
    if constexpr (HD <= 64) {
        return m;
    } else {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0) tmp4[wave] = m;
        block_sync<RAW>();
        const int t = (threadIdx.x / HD) & 1;
        const float r = fmaxf(tmp4[2 * t], tmp4[2 * t + 1]);
        block_sync<RAW>();
        return r;
    }
}

// One position of k (threads [0, HD)) and v (threads [HD, 2 HD)) of kv head
// g in the cache format: `bits` is the element (fp32 bits, bf16 bits or the
// int8 code), `scale` the int8 scale of the thread's row.  Returns the value
// read back from the cache format.  Every thread of the block must call it.
template <int KVDT, int HD, bool RAW = false>
__device__ __forceinline__ float kv_encode_head(float val, float *tmp4, uint32_t &bits, float &scale)
{
    const bool active = threadIdx.x < 2 * HD;
    float stored = 0.f;
    bits = 0u;
    scale = 0.f;
    if constexpr (KVDT == K2_F32) {
        bits = __float_as_uint(val);
        stored = val;
    } else if constexpr (KVDT == K2_BF16) {
        const uint16_t b = f32_to_bf16_rne(val);
        bits = b;
        stored = bf16_to_f32(b);
    } else {
        const float amax = kv_head_absmax<HD, RAW>(active ? fabsf(val) : 0.f, tmp4);
        const float s = amax / 127.0f;
        float q = 0.f;
        if (amax != 0.f) {
            q = rintf(val / s);
            q = fminf(fmaxf(q, -127.f), 127.f);
        }
        bits = (uint32_t)(uint8_t)(int8_t)(int)q;
        scale = amax != 0.f ? s : 0.f;
        stored = q * scale;
    }
    return active ? stored : 0.f;
}

// Write what kv_encode_head produced into slot pos of the cache (threads
// [0, 2 HD); the first thread of each row also writes the int8 scale).
template <int KVDT, int HD>
__device__ __forceinline__ void kv_write_head(uint32_t bits, float scale, void *kc, void *vc,
                                              float *ks, float *vs, int g, int cap, int pos)
{
    const int t = threadIdx.x;
    if (t >= 2 * HD) return;
    const bool is_k = t < HD;
    const int d = is_k ? t : t - HD;
    const int64_t idx = ((int64_t)g * cap + pos) * HD + d;
    if constexpr (KVDT == K2_F32) {
        (is_k ? (uint32_t *)kc : (uint32_t *)vc)[idx] = bits;
    } else if constexpr (KVDT == K2_BF16) {
        (is_k ? (uint16_t *)kc : (uint16_t *)vc)[idx] = (uint16_t)bits;
    } else {
        (is_k ? (uint8_t *)kc : (uint8_t *)vc)[idx] = (uint8_t)bits;
        if (d == 0) (is_k ? ks : vs)[(int64_t)g * cap + pos] = scale;
    }
}

// Encode and store one position (see kv_encode_head); returns the stored value.
template <int KVDT, int HD, bool RAW = false>
__device__ __forceinline__ float kv_store_head(float val, void *kc, void *vc, float *ks, float *vs,
                                               int g, int cap, int pos, float *tmp4)
{
    uint32_t bits;
    float scale;
    const float stored = kv_encode_head<KVDT, HD, RAW>(val, tmp4, bits, scale);
    kv_write_head<KVDT, HD>(bits, scale, kc, vc, ks, vs, g, cap, pos);
    return stored;
}

// ------------------------------------------------- streaming attention --
// The attention of one kv head and split, with K and V (and the int8
// scales) streamed through LDS by blocks of C::WPB waves: the block's
// positions are cut into tiles of TP positions (16 KiB of K and 16 KiB of V for head_dim 128); tiles are
// copied from HBM straight into LDS with LDS-DMA loads (global_load_lds, 16
// bytes per lane, no registers), C::NST tiles in flight, and the waves
// read them from LDS with the query heads held in registers.  A block keeps
// up to 96 KiB in flight: long contexts become bandwidth-bound.

// Optional per-block stage trace for performance work (never enabled in the
// library build): thread 0 keeps the 100 MHz real-time counter of each
// stage in LDS and writes them out when the block ends (a global store in
// between would be waited for by later waits and distort the stages).
#ifdef K2_ATTN_TRACE
static __device__ unsigned long long k2_attn_trace[4096][12];
static __shared__ unsigned long long k2_attn_trs[12];
#define K2_ATRACE(i)                                                                         \
    do {                                                                                     \
        if (threadIdx.x == 0) k2_attn_trs[i] = __builtin_amdgcn_s_memrealtime();             \
    } while (0)
#define K2_ATRACE_FLUSH()                                                                    \
    do {                                                                                     \
        const int b_ = blockIdx.y * gridDim.x + blockIdx.x;                                  \
        if (threadIdx.x == 0 && b_ < 4096)                                                   \
            for (int i_ = 0; i_ < 12; ++i_) k2_attn_trace[b_][i_] = k2_attn_trs[i_];         \
    } while (0)
#define K2_ATRACE_CLEAR()                                                                    \
    do {                                                                                     \
        if (threadIdx.x == 0)                                                                \
            for (int i_ = 0; i_ < 12; ++i_) k2_attn_trs[i_] = 0ull;                          \
    } while (0)
#else
#define K2_ATRACE(i) \
    do {         \
    } while (0)
#define K2_ATRACE_FLUSH() \
    do {              \
    } while (0)
#define K2_ATRACE_CLEAR() \
    do {              \
    } while (0)
#endif

// Block shape of the streaming attention: waves per block, tiles in flight,
// bytes per K (or V) tile.  Every attention kernel uses 8 waves and 16 KiB K
// + 16 KiB V tiles; the ring holds 3 stages for fp32 / bf16 caches (~98 KiB
// of LDS, one block per compute unit) and 2 for int8 (~66 KiB, two blocks
// per unit).  Measured at the 3.7B shape: bf16 cache, decode step with the
// position on the device 2.139 ms with 3 stages against 2.149 with 2; int8
// attention at 32k positions 28.7 us with 2 against 30.8 with 3; 8 KiB
// tiles (3 or 4 stages) were slower at 32k (35.7-36.9 us).
template <int WPB_, int NST_, int TILE_>
struct StreamCfg {
    static constexpr int WPB = WPB_, NT = WPB_ * K2_WAVE, NST = NST_, TILE = TILE_;
};
template <int KVDT>
using StreamFor = StreamCfg<8, KVDT == K2_I8 ? 2 : 3, 16384>;
constexpr int ATT_NT = StreamFor<K2_BF16>::NT;   // threads per stand-alone attention block

template <int KVDT, int HD, class C = StreamFor<KVDT>>
struct StreamGeom {
    using T = typename KVT<KVDT>::T;
    static constexpr int EPC = KVT<KVDT>::EPC;
    static constexpr int LPP = HD / EPC;                       // lanes per position
    static constexpr int PPI = K2_WAVE / LPP;                  // positions per slot
    static constexpr int ROWB = HD * (int)sizeof(T);           // bytes per cache row
    static constexpr int ROUND = C::WPB * PPI;                 // positions of one slot of every wave
    static constexpr int NSLOT = (C::TILE / (ROUND * ROWB)) > 1 ? C::TILE / (ROUND * ROWB) : 1;
    static constexpr int TP = ROUND * NSLOT;                   // positions per tile
    static constexpr int TILEB = TP * ROWB;                    // bytes of one K (or V) tile
    static constexpr int NI = TILEB / (16 * C::NT);            // 16-byte copies per thread per tile
    static constexpr int SCF = KVDT == K2_I8 ? TP : 0;         // scale floats per tile (K or V)
    static constexpr int NS = (2 * SCF + C::NT - 1) / C::NT;   // 4-byte scale copies per thread
    static constexpr int NPT = 2 * NI + NS;                    // LDS-DMA instructions per tile
    static constexpr int STAGE_F = 2 * TILEB / 4 + NS * C::NT; // floats per stage
    static_assert(NI >= 1 && NI * 16 * C::NT == TILEB, "tile copy shape");
};

template <int KVDT, int HD, int REP, class C = StreamFor<KVDT>>
__host__ __device__ constexpr int attn_stream_lds_floats()
{
    // stages (reused for the wave merge afterwards), q, new k/v, merge (m, l)
    return C::NST * StreamGeom<KVDT, HD, C>::STAGE_F + REP * HD + 2 * HD + C::WPB * REP * 2 + C::WPB;
}

// Bounded wait until *p >= need (device scope; thread 0 polls, the block
// then meets at a barrier).  Returns false, after reporting K2_EHIP in
// d_err, if the count never arrives: every caller then still runs to its end,
// so the grid always drains.
constexpr int K2_WAIT_SPIN_LIMIT = 1 << 20;
#ifndef K2_WAIT_SLEEP
#define K2_WAIT_SLEEP 1
#endif
__device__ __forceinline__ unsigned coh_load_u(const unsigned *p)
{
    return __hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool block_wait_count(const unsigned *p, unsigned need, int32_t *d_err)
{
    __shared__ int ok_s;
    if (threadIdx.x == 0) {
        int spins = 0;
        unsigned v = coh_load_u(p);
        while (v < need && ++spins < K2_WAIT_SPIN_LIMIT) {
            __builtin_amdgcn_s_sleep(K2_WAIT_SLEEP);
            v = coh_load_u(p);
        }
        ok_s = v >= need;
        if (v < need && d_err) coh_store_i(d_err, K2_EHIP);
    }
    __syncthreads();
    return ok_s != 0;
}

// The new position's cache element is returned in kv_bits / kv_scale (see
// kv_encode_head) instead of being stored: the caller writes it at the end,
// so that no wait inside the block (a barrier, or the wait the compiler
// places before LDS writes that could race an LDS-DMA) waits for its
// store.  Returns whether this block holds the new position.
template <int KVDT, int HD, int REP, bool FUSED, bool COH, class C = StreamFor<KVDT>>
__device__ __forceinline__ bool attn_stream_block(const AttnArgs &a, int g, int s, int S, float *smem,
                                                  uint32_t &kv_bits, float &kv_scale)
{
    using G = StreamGeom<KVDT, HD, C>;
    using T = typename G::T;
    constexpr int EPC = G::EPC, LPP = G::LPP, PPI = G::PPI, TP = G::TP, NSLOT = G::NSLOT;
    constexpr int WPB = C::WPB, NT = C::NT, NST = C::NST;
    static_assert(WPB * REP * HD <= NST * G::STAGE_F, "wave merge fits the stages");

    float *const stages = smem;
    float *const rest = smem + NST * G::STAGE_F;
    auto qs = reinterpret_cast<float (*)[HD]>(rest);                       // [REP][HD]
    auto newkv = reinterpret_cast<float (*)[HD]>(rest + REP * HD);         // [2][HD]
    auto red_ml = reinterpret_cast<float (*)[REP][2]>(rest + REP * HD + 2 * HD);
    float *tmp4 = rest + REP * HD + 2 * HD + WPB * REP * 2;
    auto red_o = reinterpret_cast<float (*)[REP][HD]>(stages);             // after the tiles

    const int len = a.len;
    const int j0 = s * a.chunk;
    const int j1 = min(len, j0 + a.chunk);
    const bool holds_new = FUSED && (j1 == len);
    const int jc = holds_new ? j1 - 1 : j1;        // positions read from the cache
    const int n_tiles = (jc - j0 + TP - 1) / TP;   // 0 when the block holds only the new position
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int sub = lane / LPP, cl = lane % LPP;
    const char *kb = reinterpret_cast<const char *>(reinterpret_cast<const T *>(a.kc) + (int64_t)g * a.cap * HD);
    const char *vb = reinterpret_cast<const char *>(reinterpret_cast<const T *>(a.vc) + (int64_t)g * a.cap * HD);
    const float *ksb = KVDT == K2_I8 ? a.ks + (int64_t)g * a.cap : nullptr;
    const float *vsb = KVDT == K2_I8 ? a.vs + (int64_t)g * a.cap : nullptr;
    K2_ATRACE(0);

    // q (and the new k, v): loaded first, so that waiting for them never
    // waits for the tile copies issued after them
    constexpr int QV = (REP * HD + NT - 1) / NT;
    constexpr int HALF = HD / 2;
    float qx0[QV], qx1[QV], qc[QV], qsn[QV];
    float nk0 = 0.f, nk1 = 0.f, kc0 = 0.f, ks0 = 0.f;
    auto load_qkv = [&]() {
#pragma unroll
        for (int v = 0; v < QV; ++v) {
            const int t = tid + v * NT;
            const int tt = t < REP * HD ? t : 0;
            const int hl = tt / HD, d = tt % HD, h = g * REP + hl;
            if constexpr (FUSED) {
                const float *u = a.qkv + (int64_t)h * HD;
                qx0[v] = ld1<false>(u + d % HALF);
                qx1[v] = ld1<false>(u + d % HALF + HALF);
                qc[v] = a.cos_sin[((int64_t)a.pos * HALF + d % HALF) * 2];
                qsn[v] = a.cos_sin[((int64_t)a.pos * HALF + d % HALF) * 2 + 1];
            } else {
                qx0[v] = a.q[(int64_t)h * HD + d];
                qx1[v] = qc[v] = qsn[v] = 0.f;
            }
        }
        if constexpr (FUSED) {
            if (holds_new) {
                if (tid < HD) {
                    const float *u = a.qkv + (int64_t)(a.n_qh + g) * HD;
                    nk0 = ld1<false>(u + tid % HALF);
                    nk1 = ld1<false>(u + tid % HALF + HALF);
                    kc0 = a.cos_sin[((int64_t)a.pos * HALF + tid % HALF) * 2];
                    ks0 = a.cos_sin[((int64_t)a.pos * HALF + tid % HALF) * 2 + 1];
                } else if (tid < 2 * HD) {
                    nk0 = ld1<false>(a.qkv + (int64_t)(a.n_qh + a.n_kv + g) * HD + (tid - HD));
                }
            }
        }
    };
    load_qkv();

    // tile t -> stage t % NST: K rows, V rows, then the int8 scales
    auto issue_tile = [&](int t) {
        float *st = stages + (t % NST) * G::STAGE_F;
        const int64_t p0 = j0 + (int64_t)t * TP;
        const int64_t lim = (int64_t)jc * G::ROWB - 16;         // last valid 16-byte chunk
#pragma unroll
        for (int i = 0; i < G::NI; ++i) {
            const int c = i * NT + tid;                           // 16-byte chunk of the tile
            int64_t off = p0 * G::ROWB + (int64_t)c * 16;
            off = off < lim ? off : lim;
            char *dst = reinterpret_cast<char *>(st) + (int64_t)(i * NT + wave * K2_WAVE) * 16;
            __builtin_amdgcn_global_load_lds(kb + off, dst, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vb + off, dst + G::TILEB, 16, 0, 0);
        }
        if constexpr (KVDT == K2_I8) {
#pragma unroll
            for (int i = 0; i < G::NS; ++i) {
                const int e = i * NT + tid;                       // element of [K scales | V scales]
                const bool isk = e < TP;
                int64_t p = p0 + (isk ? e : e - TP);
                p = p < jc ? p : jc - 1;
                const float *src = (e < 2 * TP) ? (isk ? ksb : vsb) + p : ksb + j0;
                float *dst = st + 2 * G::TILEB / 4 + i * NT + wave * K2_WAVE;
                __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
            }
        }
    };
#pragma unroll
    for (int t = 0; t < NST; ++t)
        if (t < n_tiles) issue_tile(t);

    // 1. query heads of this kv head, rotated (fused) and pre-scaled
#pragma unroll
    for (int v = 0; v < QV; ++v) {
        const int t = tid + v * NT;
        if (t < REP * HD) {
            const int hl = t / HD, d = t % HD;
            float val;
            if constexpr (FUSED)
                val = d < HALF ? qx0[v] * qc[v] - qx1[v] * qsn[v] : qx0[v] * qsn[v] + qx1[v] * qc[v];
            else
                val = qx0[v];
            qs[hl][d] = val * (a.scale * K2_LOG2E);   // scores in the base-2 domain
        }
    }
    // 2. fused: rotate k, store k and v at slot pos (block-uniform branch)
    if constexpr (FUSED) {
        if (holds_new) {
            float val = nk0;
            if (tid < HD) val = tid < HALF ? nk0 * kc0 - nk1 * ks0 : nk0 * ks0 + nk1 * kc0;
            const float st = kv_encode_head<KVDT, HD, true>(val, tmp4, kv_bits, kv_scale);
            if (tid < 2 * HD) newkv[tid / HD][tid % HD] = st;
        }
    }
    lds_barrier();
    K2_ATRACE(1);
    // this lane's slice of every query head, in registers
    float qv[REP][EPC], qsum[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
        qsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            qv[h][e] = qs[h][cl * EPC + e];
            qsum[h] += qv[h][e];
        }
    }

    // int8 codes are decoded as unsigned bytes u = code + 128 (one convert
    // per element); q.k = q.u - 128 sum(q) per lane, and the V sum carries
    // w = sum of the V weights to subtract 128 w at the end
    float m[REP], l[REP], acc[REP][EPC], wsum[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
        wsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
    }

    // 3. tiles: wait for tile t (later tiles may stay in flight), compute it
    //    from LDS, then reuse its stage for tile t + NST
#pragma unroll 1
    for (int t = 0; t < n_tiles; ++t) {
        const int ahead = n_tiles - 1 - t < NST - 1 ? n_tiles - 1 - t : NST - 1;
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(K2_VMCNT(2 * G::NPT));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(K2_VMCNT(G::NPT));
        else __builtin_amdgcn_s_waitcnt(K2_VMCNT(0));
        lds_barrier();
        if (t == 0) K2_ATRACE(2);
        const float *st = stages + (t % NST) * G::STAGE_F;
        const char *kt = reinterpret_cast<const char *>(st);
        const char *vt = kt + G::TILEB;
        const float *kst = st + 2 * G::TILEB / 4, *vst = kst + TP;
        const int p0 = j0 + t * TP;
        // slots of this wave with at least one cached position (a prefix of
        // the slots; wave-uniform): short chunks leave later slots empty
        int ns = 0;
#pragma unroll
        for (int n = 0; n < NSLOT; ++n)
            if (p0 + (n * WPB + wave) * PPI < jc) ns = n + 1;
        float sc[NSLOT][REP];
        int pr[NSLOT];
#pragma unroll
        for (int n = 0; n < NSLOT; ++n) {
            const int r = (n * WPB + wave) * PPI + sub;            // row within the tile
            pr[n] = r;
            if (n >= ns) {
#pragma unroll
                for (int h = 0; h < REP; ++h) sc[n][h] = -INFINITY;
                continue;
            }
            float kv[EPC];
            kv_decode_u<KVDT>(*reinterpret_cast<const k2_u4 *>(kt + r * G::ROWB + cl * 16), kv);
            const bool valid = p0 + r < jc;
            const float ksc = (KVDT == K2_I8) ? kst[r] : 1.0f;
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                float p = (KVDT == K2_I8) ? -128.0f * qsum[h] : 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) p += qv[h][e] * kv[e];
                p = group_sum<LPP>(p) * ksc;
                sc[n][h] = valid ? p : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            float mx = sc[0][h];
#pragma unroll
            for (int n = 1; n < NSLOT; ++n) mx = fmaxf(mx, sc[n][h]);
            // lazy rescaling: the reference m (wave-uniform) moves only when
            // a score passes it by more than ATT_SLACK (base 2), so a tile
            // mostly skips the wave maximum; the weights 2^(s - m) stay
            // <= 2^ATT_SLACK, and any reference gives the same softmax
            if (__builtin_amdgcn_ballot_w64(mx > m[h] + ATT_SLACK) != 0) {   // uniform
                mx = wave_max(mx);
                const float corr = k2_exp2(m[h] - mx);   // m = -inf gives 0
                l[h] *= corr;
                wsum[h] *= corr;
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[h][e] *= corr;
                m[h] = mx;
            }
        }
#pragma unroll
        for (int n = 0; n < NSLOT; ++n) {
            if (p0 + pr[n] < jc) {
                float vv[EPC];
                kv_decode_u<KVDT>(*reinterpret_cast<const k2_u4 *>(vt + pr[n] * G::ROWB + cl * 16), vv);
                const float vsc = (KVDT == K2_I8) ? vst[pr[n]] : 1.0f;
#pragma unroll
                for (int h = 0; h < REP; ++h) {
                    const float p = k2_exp2(sc[n][h] - m[h]);
                    l[h] += p;
                    const float pv = p * vsc;
                    if constexpr (KVDT == K2_I8) wsum[h] += pv;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[h][e] += pv * vv[e];
                }
            }
        }
        lds_barrier();                               // every wave is done with stage t % NST
        if (t + NST < n_tiles) issue_tile(t + NST);
    }
    K2_ATRACE(3);
    if constexpr (KVDT == K2_I8) {
#pragma unroll
        for (int h = 0; h < REP; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] -= 128.0f * wsum[h];
    }
    // the new position (fused): wave 0, values from LDS (read by every lane;
    // only sub-group 0 adds them)
    if (holds_new && wave == 0) {
        float nv[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) nv[e] = newkv[1][cl * EPC + e];
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            float p = 0.f;
            for (int d = lane; d < HD; d += K2_WAVE) p += qs[h][d] * newkv[0][d];
            const float snew = wave_sum(p);
            const float mn = fmaxf(m[h], snew);
            const float corr = k2_exp2(m[h] - mn);       // m = -inf gives 0
            const float pw = sub == 0 ? k2_exp2(snew - mn) : 0.f;
            l[h] = l[h] * corr + pw;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] = acc[h][e] * corr + pw * nv[e];
            m[h] = mn;
        }
    }
    K2_ATRACE(7);
    // 4. sum over the position sub-groups of the wave (m is the same across
    // the wave): lane swaps and rotations, no LDS
#pragma unroll
    for (int h = 0; h < REP; ++h) l[h] = subgroup_sum<LPP>(l[h]);
    if constexpr (LPP >= 8 && LPP <= 32 && (REP * EPC) % PPI == 0) {
        // reduce-scatter: every lane ends with REP*EPC/PPI of the sums
        constexpr int NV = REP * EPC, NJ = NV / PPI;
        float v[NV];
#pragma unroll
        for (int h = 0; h < REP; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) v[h * EPC + e] = acc[h][e];
        group_reduce_scatter<NV, LPP>(v, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int k = j + NJ * sub;            // flat (head, element) index
            red_o[wave][k / EPC][cl * EPC + k % EPC] = v[j];
        }
    } else {
#pragma unroll
        for (int h = 0; h < REP; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] = subgroup_sum<LPP>(acc[h][e]);
        if (sub == 0) {
#pragma unroll
            for (int h = 0; h < REP; ++h)
#pragma unroll
                for (int e = 0; e < EPC; ++e) red_o[wave][h][cl * EPC + e] = acc[h][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < REP; ++h) { red_ml[wave][h][0] = m[h]; red_ml[wave][h][1] = l[h]; }
    }
    __syncthreads();
    K2_ATRACE(8);

    // 5. combine the waves; output directly (one split) or publish a partial
    const int64_t pbase = ((int64_t)g * S + s) * REP;
    for (int t = tid; t < REP * HD; t += NT) {
        const int h = t / HD, d = t % HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WPB; ++w) M = fmaxf(M, red_ml[w][h][0]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < WPB; ++w) {
            const float mw = red_ml[w][h][0];
            const float f = (mw == -INFINITY) ? 0.f : k2_exp2(mw - M);
            L += f * red_ml[w][h][1];
            o += f * red_o[w][h][d];
        }
        if (S == 1) {
            st1<COH>(a.out + (int64_t)(g * REP + h) * HD + d, o / L);
        } else {
            st1<COH>(a.part + (pbase + h) * HD + d, o);
            if (d == 0) {
                // the combine works with natural-log maxima
                st1<COH>(a.part_ml + (pbase + h) * 2, M * K2_LN2);
                st1<COH>(a.part_ml + (pbase + h) * 2 + 1, L);
            }
        }
    }
    return holds_new;
}

template <int REP, int NTH = K2_BLOCK>
__host__ __device__ constexpr int combine_lds_floats()
{
    return ((2 * K2_ATTN_MAX_SPLITS * REP + 2 * REP + 3) & ~3) + NTH * 4;
}

// Combine for kv head g (a block of NTH threads; every thread calls it):
// M = max_s m_s, L = sum_s l_s e^(m_s - M), out = sum_s o_s e^(m_s - M) / L
// (a fixed summation order, so the result does not depend on which block
// combines).  Float4 column c of the head's
// REP*HD/4 columns belongs to threads c, c + C4, ...; every thread issues
// its first NB partial float4s and its (m, l) pairs before it uses any of
// them, so that (for S <= NB * threads per column) the whole combine costs
// one memory round trip.
template <int HD, int REP, bool COH, int NTH = K2_BLOCK>
__device__ __forceinline__ void attn_combine_block(const AttnArgs &a, int g, float *smem)
{
    constexpr int C4 = REP * HD / 4;                     // float4 columns of a split
    constexpr int TPC = C4 >= NTH ? 1 : NTH / C4;        // threads per column
    constexpr int CPT = C4 >= NTH ? C4 / NTH : 1;        // columns per thread
    constexpr int NB = 16;                               // loads in flight per batch
    static_assert(C4 % NTH == 0 || NTH % C4 == 0, "combine shape");
    auto fm = reinterpret_cast<float (*)[REP]>(smem);    // [MAX_SPLITS][REP] maxima
    auto fl = reinterpret_cast<float (*)[REP]>(smem + K2_ATTN_MAX_SPLITS * REP);   // sums
    float *Linv = smem + 2 * K2_ATTN_MAX_SPLITS * REP;                            // [REP]
    float4 *part4 = reinterpret_cast<float4 *>(smem + ((2 * K2_ATTN_MAX_SPLITS * REP + 2 * REP + 3) & ~3));
    const int S = a.S, tid = threadIdx.x;
    const float *ml = a.part_ml + (int64_t)g * S * REP * 2;
    const float *po = a.part + (int64_t)g * S * REP * HD;
    const int c0 = (C4 >= NTH) ? tid : tid % C4;          // first float4 column
    const int q0 = (C4 >= NTH) ? 0 : tid / C4;            // first split
    // 1. every load of the first batch, then the (m, l) pairs (q0 is
    // uniform over a wave, so the guards do not diverge; no load is issued
    // past the last split: repeated reads of one line from every thread
    // would all queue on one memory channel)
    float4 v[CPT][NB];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc)
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int q = q0 + i * TPC;
            v[cc][i] = q < S ? ld4<COH>(po, (q * C4 + c0 + cc * NTH) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    for (int t = tid; t < S * REP; t += NTH) {
        const float m = ld1<COH>(ml + (int64_t)t * 2), l = ld1<COH>(ml + (int64_t)t * 2 + 1);
        fm[t / REP][t % REP] = m;
        fl[t / REP][t % REP] = l;
    }
    __syncthreads();
    K2_ATRACE(9);
    // 2. per head (one wave each): M, the split weights e^(m_s - M) in place
    // of the maxima, and 1 / L
    {
        const int wave = tid >> 6, lane = tid & 63;
        for (int h = wave; h < REP; h += NTH / K2_WAVE) {
            float M = -INFINITY;
            for (int q = lane; q < S; q += K2_WAVE) M = fmaxf(M, fm[q][h]);
            M = wave_max(M);
            float L = 0.f;
            for (int q = lane; q < S; q += K2_WAVE) {
                const float mq = fm[q][h];
                const float w = mq == -INFINITY ? 0.f : expf(mq - M);
                fm[q][h] = w;
                L += w * fl[q][h];
            }
            L = wave_sum(L);
            if (lane == 0) Linv[h] = 1.0f / L;
        }
    }
    __syncthreads();
    K2_ATRACE(10);
    // 3. weighted sums of the partials
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
        const int c = c0 + cc * NTH;
        const int h = c * 4 / HD;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int qb = q0; qb < S; qb += TPC * NB) {
            if (qb != q0) {                                // later batches (S > NB * TPC)
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const int q = qb + i * TPC;
                    v[cc][i] = q < S ? ld4<COH>(po, (q * C4 + c) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int q = qb + i * TPC;
                const float w = q < S ? fm[q][h] : 0.f;
                o.x += w * v[cc][i].x; o.y += w * v[cc][i].y; o.z += w * v[cc][i].z; o.w += w * v[cc][i].w;
            }
        }
        if constexpr (TPC > 1) {
            part4[tid] = o;
            __syncthreads();
            if (tid < C4) {
                o = part4[tid];
#pragma unroll
                for (int k = 1; k < TPC; ++k) {
                    const float4 u = part4[tid + k * C4];
                    o.x += u.x; o.y += u.y; o.z += u.z; o.w += u.w;
                }
            }
        }
        if (tid < C4 || C4 >= NTH) {
            const float li = Linv[h];
            float *out = a.out + (int64_t)g * REP * HD + c * 4;
            st1<COH>(out, o.x * li);
            st1<COH>(out + 1, o.y * li);
            st1<COH>(out + 2, o.z * li);
            st1<COH>(out + 3, o.w * li);
        }
    }
}

// Position taken from device memory (a.d_pos set): pos, len, chunk and the
// split count S follow from *d_pos by the rule of attn_splits on the host
// (chunk = ceil(len / target) clamped to [K2_ATTN_MIN_CHUNK,
// K2_ATTN_MAX_CHUNK], target = K2_ATTN_TARGET_BLOCKS / n_kv), with the chunk
// raised where needed so that S never exceeds Sg, the grid's split extent
// (a longer range per block: the kernels take any chunk).
// Returns false for a position outside [0, cap): the first block reports
// K2_ERANGE in d_err and every block leaves without writing.
__device__ __forceinline__ bool attn_resolve_pos(AttnArgs &a, int Sg)
{
    if (!a.d_pos) return true;
    const int p = *a.d_pos;            // written by an earlier kernel of the stream
    if (p < 0 || p >= a.cap) {
        if (a.d_err && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) coh_store_i(a.d_err, K2_ERANGE);
        return false;
    }
    a.pos = p;
    a.len = p + 1;
    int target = K2_ATTN_TARGET_BLOCKS / a.n_kv;
    if (target < 1) target = 1;
    int c = (a.len + target - 1) / target;
    c = c < K2_ATTN_MIN_CHUNK ? K2_ATTN_MIN_CHUNK : c;
    c = c > K2_ATTN_MAX_CHUNK ? K2_ATTN_MAX_CHUNK : c;
    const int cg = (a.len + Sg - 1) / Sg;
    c = c > cg ? c : cg;
    a.chunk = c;
    a.S = (a.len + c - 1) / c;
    return true;
}

// Blocks with blockIdx.y >= n_kv read the weight range pf, split evenly over
// them in 16-byte units, with plain loads (which allocate in the memory-side
// cache), and exit.  They share no state with the attention blocks; the
// kernel's duration bounds theirs.
__device__ __forceinline__ void attn_prefetch_block(const AttnArgs &a)
{
    const int64_t nblk = (int64_t)gridDim.x * (gridDim.y - a.n_kv);
    const int64_t b = (int64_t)(blockIdx.y - a.n_kv) * gridDim.x + blockIdx.x;
    const int64_t units = a.pf_bytes >> 4;
    const int64_t per = (units + nblk - 1) / nblk;
    const int64_t lo = b * per, hi = lo + per < units ? lo + per : units;
    const k2_u4 *p = reinterpret_cast<const k2_u4 *>(a.pf);
    constexpr int D = 8;
    uint32_t acc = 0u;
    for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)D * blockDim.x) {
        k2_u4 v[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t j = i + (int64_t)d * blockDim.x;
            v[d] = p[j < hi ? j : lo];                 // clamp: in-range, branch-free
        }
#pragma unroll
        for (int d = 0; d < D; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    asm volatile("" ::"v"(acc));                      // keep the loads
}

// One launch: every block attends over its split; with several splits the
// last block of each kv head to finish (an arrival counter, reset by that
// block) combines the partials of the head.  No block waits for another.
template <int KVDT, int HD, int REP, bool FUSED>
__global__ __launch_bounds__(ATT_NT) void attn_kernel(const AttnArgs a0)
{
    constexpr int NA = attn_stream_lds_floats<KVDT, HD, REP>(), NC = combine_lds_floats<REP, ATT_NT>();
    extern __shared__ float4 lds4[];
    float *smem = reinterpret_cast<float *>(lds4);
    static_assert(NA >= NC, "combine fits the attention LDS");
    __shared__ int last;
    if ((int)blockIdx.y >= a0.n_kv) {
        attn_prefetch_block(a0);
        return;
    }
    AttnArgs a = a0;
    if (!attn_resolve_pos(a, gridDim.x)) return;
    if ((int)blockIdx.x >= a.S) return;            // device split count below the grid's
    const int g = blockIdx.y, S = a.S;
    K2_ATRACE_CLEAR();
    uint32_t kv_bits = 0u;
    float kv_scale = 0.f;
    const bool holder = attn_stream_block<KVDT, HD, REP, FUSED, true>(a, g, blockIdx.x, S, smem, kv_bits,
                                                                      kv_scale);
    K2_ATRACE(4);
    if (S > 1) {
        __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores completed
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(a.head_cnt + g, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            last = old == (unsigned)S - 1;
            if (last) __hip_atomic_store(a.head_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        K2_ATRACE(5);
        if (last) {
            attn_combine_block<HD, REP, true, ATT_NT>(a, g, smem);
            K2_ATRACE(6);
        }
    }
    // the new position's K/V: no other block of this launch reads slot pos
    // (the block holding it used the values from LDS)
    if (FUSED && holder) kv_write_head<KVDT, HD>(kv_bits, kv_scale, a.kc, a.vc, a.ks, a.vs, g, a.cap, a.pos);
    K2_ATRACE_FLUSH();
}

// Attention of T consecutive query positions (a prefill chunk) in one
// launch, grid (S, n_kv, T): slice t (blockIdx.z) is the query of position
// a.len - T + t over [0, that position] -- the chunk's K/V rows are already
// in the cache and q is already rotated (rope_append_rows_kernel).  Every
// slice has its own split count S_t <= gridDim.x (blocks past it exit at
// once), its own partials and its own arrival counters; within a slice the
// blocks run exactly as in attn_kernel.
template <int KVDT, int HD, int REP>
__global__ __launch_bounds__(ATT_NT) void attn_rows_kernel(const AttnArgs a0, int n_rows, int64_t part_stride,
                                                           int64_t ml_stride)
{
    extern __shared__ float4 lds4[];
    float *smem = reinterpret_cast<float *>(lds4);
    __shared__ int last;
    const int t = blockIdx.z, g = blockIdx.y, s = blockIdx.x;
    AttnArgs a = a0;
    a.len = a0.len - (n_rows - 1 - t);
    a.pos = a.len - 1;
    const int S = (a.len + a.chunk - 1) / a.chunk;
    if (s >= S) return;
    a.S = S;
    a.q = a0.q + (int64_t)t * a0.n_qh * HD;
    a.out = a0.out + (int64_t)t * a0.n_qh * HD;
    a.part = a0.part + t * part_stride;
    a.part_ml = a0.part_ml + t * ml_stride;
    a.head_cnt = a0.head_cnt + (int64_t)t * a0.n_kv;
    uint32_t kv_bits = 0u;
    float kv_scale = 0.f;
    attn_stream_block<KVDT, HD, REP, false, true>(a, g, s, S, smem, kv_bits, kv_scale);
    if (S > 1) {
        __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores completed
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(a.head_cnt + g, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            last = old == (unsigned)S - 1;
            if (last) __hip_atomic_store(a.head_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (last) attn_combine_block<HD, REP, true, ATT_NT>(a, g, smem);
    }
}

// RoPE and cache append for the T rows of a prefill chunk, grid (n_kv, T),
// K2_BLOCK threads: block (g, t) takes row t of qkv [T][(n_qh + 2 n_kv) HD]
// at position pos0 + t, rotates the REP query heads of kv head g into
// qrot [T][n_qh][HD] and k of head g, and stores k and v of head g at that
// slot in the cache format (kv_store_head: the same encoding as every other
// append).
template <int KVDT, int HD>
__global__ __launch_bounds__(K2_BLOCK) void rope_append_rows_kernel(const float *qkv, const float *cs,
                                                                    float *qrot, void *kc, void *vc,
                                                                    float *ks, float *vs, int n_qh,
                                                                    int n_kv, int cap, int pos0)
{
    __shared__ float tmp4[K2_WAVES_PER_BLOCK];
    constexpr int HALF = HD / 2;
    const int g = blockIdx.x, t = blockIdx.y, tid = threadIdx.x, rep = n_qh / n_kv;
    const int pos = pos0 + t;
    const float *row = qkv + (int64_t)t * (n_qh + 2 * n_kv) * HD;
    const float *csp = cs + (int64_t)pos * HALF * 2;
    for (int e = tid; e < rep * HD; e += K2_BLOCK) {
        const int h = g * rep + e / HD, d = e % HD, i = d % HALF;
        const float *u = row + (int64_t)h * HD;
        const float c = csp[i * 2], sn = csp[i * 2 + 1], x0 = u[i], x1 = u[i + HALF];
        qrot[((int64_t)t * n_qh + h) * HD + d] = d < HALF ? x0 * c - x1 * sn : x0 * sn + x1 * c;
    }
    float val = 0.f;
    if (tid < HD) {
        const float *u = row + (int64_t)(n_qh + g) * HD;
        const int i = tid % HALF;
        const float c = csp[i * 2], sn = csp[i * 2 + 1], x0 = u[i], x1 = u[i + HALF];
        val = tid < HALF ? x0 * c - x1 * sn : x0 * sn + x1 * c;
    } else if (tid < 2 * HD) {
        val = row[(int64_t)(n_qh + n_kv + g) * HD + tid - HD];
    }
    kv_store_head<KVDT, HD>(val, kc, vc, ks, vs, g, cap, pos, tmp4);
}

// Standalone store of one position (k, v already rotated), grid = n_kv.
template <int KVDT, int HD>
__global__ __launch_bounds__(K2_BLOCK) void kv_append_kernel(const float *k, const float *v,
                                                              void *kc, void *vc, float *ks,
                                                              float *vs, int cap, int pos)
{
    __shared__ float tmp4[K2_WAVES_PER_BLOCK];
    const int g = blockIdx.x, t = threadIdx.x;
    float val = 0.f;
    if (t < HD) val = k[(int64_t)g * HD + t];
    else if (t < 2 * HD) val = v[(int64_t)g * HD + t - HD];
    kv_store_head<KVDT, HD>(val, kc, vc, ks, vs, g, cap, pos, tmp4);
}

}  // namespace k2
