// attn_impl.h -- device code of the split-K GQA decode attention (included
// by attn.hip for the standalone kernels and by the persistent step kernel).
//
// Semantics ([k2-burn] "Model shape": GQA with 4x KV repeat; "Limitations":
// plain SDPA, softmax in fp32; "KV cache storage": fp32 / bf16 / symmetric
// int8 with one scale per head_dim block):
//   out[h] = softmax_j(q_h . K_hat[g][j] * scale) V_hat[g][j],  g = h / rep,
// over positions j in [0, len).
//
// Grid: (S splits, n_kv heads); block = 256 threads.  Block (s, g) handles
// positions [s*chunk, min(len, (s+1)*chunk)) for the rep query heads of kv
// head g:
//   1. the rep query heads are rotated (fused form) and scaled into LDS;
//   2. each wave streams its positions: a K (and V) row of head_dim values is
//      split over LPP lanes that each load 16 bytes, so one wave instruction
//      covers 64/LPP positions; the K and V loads of NL such slots are issued
//      together before any arithmetic; the int8 per-position scale multiplies
//      the finished dot product and is folded into the probability for V;
//   3. each wave keeps an online fp32 softmax (running max, rescaled sum and
//      accumulator); the four waves are merged through LDS;
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

// Largest |x| over the head_dim values of k (threads [0, HD)) and of v
// (threads [HD, 2 HD)); every thread must call it.
template <int HD>
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
        __syncthreads();
        const int t = (threadIdx.x / HD) & 1;
        const float r = fmaxf(tmp4[2 * t], tmp4[2 * t + 1]);
        __syncthreads();
        return r;
    }
}

// Store one position of k (threads [0, HD)) and v (threads [HD, 2 HD)) for kv
// head g into the cache; returns (through `stored`) the value read back from
// the cache format.  Every thread of the block must call it.
template <int KVDT, int HD>
__device__ __forceinline__ float kv_store_head(float val, void *kc, void *vc, float *ks, float *vs,
                                               int g, int cap, int pos, float *tmp4)
{
    const int t = threadIdx.x;
    const bool is_k = t < HD, active = t < 2 * HD;
    const int d = is_k ? t : t - HD;
    const int64_t idx = ((int64_t)g * cap + pos) * HD + d;
    float stored = 0.f;
    if constexpr (KVDT == K2_F32) {
        if (active) {
            (is_k ? (float *)kc : (float *)vc)[idx] = val;
            stored = val;
        }
    } else if constexpr (KVDT == K2_BF16) {
        if (active) {
            const uint16_t b = f32_to_bf16_rne(val);
            (is_k ? (uint16_t *)kc : (uint16_t *)vc)[idx] = b;
            stored = bf16_to_f32(b);
        }
    } else {
        const float amax = kv_head_absmax<HD>(active ? fabsf(val) : 0.f, tmp4);
        if (active) {
            const float s = amax / 127.0f;
            float q = 0.f;
            if (amax != 0.f) {
                q = rintf(val / s);
                q = fminf(fmaxf(q, -127.f), 127.f);
            }
            (is_k ? (int8_t *)kc : (int8_t *)vc)[idx] = (int8_t)(int)q;
            if (d == 0) (is_k ? ks : vs)[(int64_t)g * cap + pos] = amax != 0.f ? s : 0.f;
            stored = q * (amax != 0.f ? s : 0.f);
        }
    }
    return stored;
}

// LDS of attn_block, carved from a float buffer of attn_lds_floats<...>()
template <int HD, int REP, int WPB>
__host__ __device__ constexpr int attn_lds_floats()
{
    return REP * HD + 2 * HD + WPB * REP * HD + WPB * REP * 2 + WPB;
}

// One block of the attention: kv head g, split s of S (positions
// [s*chunk, min(len, (s+1)*chunk))).  Every thread of the block calls it.
// COH: partials and outputs go to other blocks of the same grid: they are
// stored at device scope, and the combine reads partials at device scope
// (the partial buffer is reused by every layer, so a plain load could hit a
// stale L2 line).  LEAN: fewer registers (half the slots in flight, q read
// from LDS) for kernels whose other phases set the register budget.
template <int KVDT, int HD, int REP, bool FUSED, int WPB, bool COH, bool LEAN = false>
__device__ __forceinline__ void attn_block(const AttnArgs &a, int g, int s, int S, float *smem)
{
    using T = typename KVT<KVDT>::T;
    constexpr int EPC = KVT<KVDT>::EPC;
    constexpr int LPP = HD / EPC;                  // lanes per position
    constexpr int PPI = K2_WAVE / LPP;             // positions per wave slot
    constexpr int NL = LEAN ? (EPC >= 16 ? 1 : 2) : (EPC >= 16 ? 2 : 4);   // slots per wave per iteration
    constexpr int NT = WPB * K2_WAVE;              // threads per block
    static_assert(LPP >= 1 && LPP <= K2_WAVE, "head_dim / dtype");

    auto qs = reinterpret_cast<float (*)[HD]>(smem);                         // [REP][HD]
    auto newkv = reinterpret_cast<float (*)[HD]>(smem + REP * HD);           // [2][HD]
    auto red_o = reinterpret_cast<float (*)[REP][HD]>(smem + REP * HD + 2 * HD);  // [WPB][REP][HD]
    auto red_ml = reinterpret_cast<float (*)[REP][2]>(smem + REP * HD + 2 * HD + WPB * REP * HD);
    float *tmp4 = smem + REP * HD + 2 * HD + WPB * REP * HD + WPB * REP * 2;
    const int len = a.len;
    const int j0 = s * a.chunk;
    const int j1 = min(len, j0 + a.chunk);
    const bool holds_new = FUSED && (j1 == len);
    const int jc = holds_new ? j1 - 1 : j1;        // positions read from the cache
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int sub = lane / LPP, cl = lane % LPP;

    const T *__restrict__ kbase = reinterpret_cast<const T *>(a.kc) + (int64_t)g * a.cap * HD;
    const T *__restrict__ vbase = reinterpret_cast<const T *>(a.vc) + (int64_t)g * a.cap * HD;
    // The K and V rows of the first iteration do not depend on q: issue them
    // first (unconditionally, at a clamped valid position) so that they are in
    // flight while q is rotated and the new position is appended.
    k2_u4 kw[NL], vw[NL];
    int jn[NL];
    auto issue_kv = [&](int base) {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            const int j = base + (n * WPB + wave) * PPI + sub;
            jn[n] = j;
            const int jj = j < jc ? j : j0;
            kw[n] = *reinterpret_cast<const k2_u4 *>(kbase + (int64_t)jj * HD + cl * EPC);
            vw[n] = *reinterpret_cast<const k2_u4 *>(vbase + (int64_t)jj * HD + cl * EPC);
        }
    };
    issue_kv(j0);

    // 1. query heads of this kv head, rotated (fused) and pre-scaled
    for (int t = tid; t < REP * HD; t += NT) {
        const int hl = t / HD, d = t % HD, h = g * REP + hl;
        float val;
        if constexpr (FUSED) {
            constexpr int half = HD / 2;
            const float *u = a.qkv + (int64_t)h * HD;
            const int i = d % half;
            const float c = a.cos_sin[((int64_t)a.pos * half + i) * 2];
            const float sn = a.cos_sin[((int64_t)a.pos * half + i) * 2 + 1];
            const float x0 = u[i], x1 = u[i + half];
            val = d < half ? x0 * c - x1 * sn : x0 * sn + x1 * c;
        } else {
            val = a.q[(int64_t)h * HD + d];
        }
        qs[hl][d] = val * a.scale;
    }
    // 2. fused: rotate k, store k and v at slot pos (block-uniform branch)
    if constexpr (FUSED) {
        if (holds_new) {
            constexpr int half = HD / 2;
            float val = 0.f;
            if (tid < HD) {
                const float *u = a.qkv + (int64_t)(a.n_qh + g) * HD;
                const int d = tid, i = d % half;
                const float c = a.cos_sin[((int64_t)a.pos * half + i) * 2];
                const float sn = a.cos_sin[((int64_t)a.pos * half + i) * 2 + 1];
                const float x0 = u[i], x1 = u[i + half];
                val = d < half ? x0 * c - x1 * sn : x0 * sn + x1 * c;
            } else if (tid < 2 * HD) {
                val = a.qkv[(int64_t)(a.n_qh + a.n_kv + g) * HD + (tid - HD)];
            }
            const float st = kv_store_head<KVDT, HD>(val, a.kc, a.vc, a.ks, a.vs, g, a.cap, a.pos, tmp4);
            if (tid < 2 * HD) newkv[tid / HD][tid % HD] = st;
        }
    }
    __syncthreads();

    const float *__restrict__ ksb = a.ks + (int64_t)g * a.cap;
    const float *__restrict__ vsb = a.vs + (int64_t)g * a.cap;

    // q slice of this lane: in registers when small, else read from LDS at use
    constexpr bool QREG = !LEAN && REP * EPC <= 32;
    float qv[QREG ? REP : 1][QREG ? EPC : 1];
    if constexpr (QREG) {
#pragma unroll
        for (int h = 0; h < REP; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) qv[h][e] = qs[h][cl * EPC + e];
    }

    // 3. per-wave online softmax over the slots of this wave: slot n of
    //    iteration it covers positions j0 + ((it*NL + n)*WPB + wave)*PPI + [0, PPI)
    float m[REP], l[REP], acc[REP][EPC];
#pragma unroll
    for (int h = 0; h < REP; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
    }
    for (int base = j0; base < jc; base += NL * WPB * PPI) {
        // take this iteration's rows, then put the next iteration's loads in
        // flight before any arithmetic (double buffering)
        k2_u4 kcur[NL], vcur[NL];
        int jcur[NL];
#pragma unroll
        for (int n = 0; n < NL; ++n) { kcur[n] = kw[n]; vcur[n] = vw[n]; jcur[n] = jn[n]; }
        if (base + NL * WPB * PPI < jc) issue_kv(base + NL * WPB * PPI);
        float sc[NL][REP];
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            float kv[EPC];
            kv_decode<KVDT>(kcur[n], kv);
            const bool valid = jcur[n] < jc;
            const float ksc = (KVDT == K2_I8 && valid) ? ksb[jcur[n]] : 1.0f;
#pragma unroll
            for (int h = 0; h < REP; ++h) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    if constexpr (QREG) p += qv[h][e] * kv[e];
                    else p += qs[h][cl * EPC + e] * kv[e];
                }
                p = group_sum<LPP>(p) * ksc;
                sc[n][h] = valid ? p : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            float mx = sc[0][h];
#pragma unroll
            for (int n = 1; n < NL; ++n) mx = fmaxf(mx, sc[n][h]);
            mx = wave_max(mx);
            const float mn = fmaxf(m[h], mx);
            // mn is finite here: the first iteration of every wave that runs
            // holds at least one valid position (base < jc for slot 0 of wave 0;
            // other waves may see none, handled below)
            const float corr = (mn == -INFINITY) ? 1.0f : expf(m[h] - mn);
            l[h] *= corr;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] *= corr;
            m[h] = mn;
        }
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            if (jcur[n] < jc) {
                float vv[EPC];
                kv_decode<KVDT>(vcur[n], vv);
                const float vsc = (KVDT == K2_I8) ? vsb[jcur[n]] : 1.0f;
#pragma unroll
                for (int h = 0; h < REP; ++h) {
                    const float p = expf(sc[n][h] - m[h]);
                    l[h] += p;
                    const float pv = p * vsc;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[h][e] += pv * vv[e];
                }
            }
        }
    }
    // the new position (fused): wave 0, values from LDS
    if (holds_new && wave == 0) {
#pragma unroll
        for (int h = 0; h < REP; ++h) {
            float p = 0.f;
            for (int d = lane; d < HD; d += K2_WAVE) p += qs[h][d] * newkv[0][d];
            const float snew = wave_sum(p);
            const float mn = fmaxf(m[h], snew);
            const float corr = expf(m[h] - mn);          // m = -inf gives 0
            const float pn = expf(snew - mn);
            l[h] = l[h] * corr + (sub == 0 ? pn : 0.f);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                acc[h][e] = acc[h][e] * corr + (sub == 0 ? pn * newkv[1][cl * EPC + e] : 0.f);
            m[h] = mn;
        }
    }
    // 4. sum over the position sub-groups of the wave (same m across the wave)
#pragma unroll
    for (int h = 0; h < REP; ++h) {
#pragma unroll
        for (int o = LPP; o < K2_WAVE; o <<= 1) l[h] += __shfl_xor(l[h], o, K2_WAVE);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            float v = acc[h][e];
#pragma unroll
            for (int o = LPP; o < K2_WAVE; o <<= 1) v += __shfl_xor(v, o, K2_WAVE);
            acc[h][e] = v;
        }
    }
    if (sub == 0) {
#pragma unroll
        for (int h = 0; h < REP; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) red_o[wave][h][cl * EPC + e] = acc[h][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < REP; ++h) { red_ml[wave][h][0] = m[h]; red_ml[wave][h][1] = l[h]; }
    }
    __syncthreads();

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
            const float f = (mw == -INFINITY) ? 0.f : expf(mw - M);
            L += f * red_ml[w][h][1];
            o += f * red_o[w][h][d];
        }
        if (S == 1) {
            st1<COH>(a.out + (int64_t)(g * REP + h) * HD + d, o / L);
        } else {
            st1<COH>(a.part + (pbase + h) * HD + d, o);
            if (d == 0) {
                st1<COH>(a.part_ml + (pbase + h) * 2, M);
                st1<COH>(a.part_ml + (pbase + h) * 2 + 1, L);
            }
        }
    }
}

template <int REP>
__host__ __device__ constexpr int combine_lds_floats()
{
    return K2_ATTN_MAX_SPLITS * REP + 2 * REP;
}

// Combine for kv head g (a block of K2_BLOCK threads; every thread calls it).
template <int HD, int REP, bool COH>
__device__ __forceinline__ void attn_combine_block(const AttnArgs &a, int g, float *smem)
{
    auto f = reinterpret_cast<float (*)[REP]>(smem);                         // [MAX_SPLITS][REP]
    float *Mh = smem + K2_ATTN_MAX_SPLITS * REP, *Linv = Mh + REP;
    const int S = a.S, tid = threadIdx.x;
    const float *ml = a.part_ml + (int64_t)g * S * REP * 2;
    for (int t = tid; t < S * REP; t += K2_BLOCK) f[t / REP][t % REP] = ld1<COH>(ml + (int64_t)t * 2);
    __syncthreads();
    if (tid < REP) {
        float M = -INFINITY;
        for (int q = 0; q < S; ++q) M = fmaxf(M, f[q][tid]);
        Mh[tid] = M;
    }
    __syncthreads();
    for (int t = tid; t < S * REP; t += K2_BLOCK) f[t / REP][t % REP] = expf(f[t / REP][t % REP] - Mh[t % REP]);
    __syncthreads();
    if (tid < REP) {
        float L = 0.f;
        for (int q = 0; q < S; ++q) L += f[q][tid] * ld1<COH>(ml + ((int64_t)q * REP + tid) * 2 + 1);
        Linv[tid] = 1.0f / L;
    }
    __syncthreads();
    for (int t = tid; t < REP * HD; t += K2_BLOCK) {
        const int h = t / HD, d = t % HD;
        const float *po = a.part + ((int64_t)g * S * REP + h) * HD + d;
        float o = 0.f;
        int q = 0;
        for (; q + 8 <= S; q += 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = ld1<COH>(po + (int64_t)(q + i) * REP * HD);
#pragma unroll
            for (int i = 0; i < 8; ++i) o += f[q + i][h] * v[i];
        }
        for (; q < S; ++q) o += f[q][h] * ld1<COH>(po + (int64_t)q * REP * HD);
        st1<COH>(a.out + (int64_t)(g * REP + h) * HD + d, o * Linv[h]);
    }
}

// One launch: every block attends over its split; with several splits the
// last block of each kv head to finish (an arrival counter, reset by that
// block) combines the partials of the head.  No block waits for another.
template <int KVDT, int HD, int REP, bool FUSED, int WPB>
__global__ __launch_bounds__(WPB * K2_WAVE) void attn_kernel(const AttnArgs a)
{
    constexpr int NA = attn_lds_floats<HD, REP, WPB>(), NC = combine_lds_floats<REP>();
    __shared__ float smem[NA > NC ? NA : NC];
    __shared__ int last;
    const int g = blockIdx.y, S = gridDim.x;
    attn_block<KVDT, HD, REP, FUSED, WPB, true>(a, g, blockIdx.x, S, smem);
    if (S == 1) return;
    __builtin_amdgcn_s_waitcnt(0);                 // this thread's partial stores completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.head_cnt + g, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last = old == (unsigned)S - 1;
        if (last) __hip_atomic_store(a.head_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (last) attn_combine_block<HD, REP, true>(a, g, smem);
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
