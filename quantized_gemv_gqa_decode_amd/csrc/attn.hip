// attn.hip -- split-K GQA decode attention for gfx950, with the RoPE and
// KV-cache append of the new position fused in.
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
//      every block publishes (max, sum, unnormalised o) and a second small
//      kernel combines the S partials of each kv head in split order (fixed
//      order: the result is run-to-run deterministic).
// Fused form: the block holding the new position `pos` also rotates k, stores
// k and v at slot pos in the cache format, and uses the stored (dequantized)
// values for that position from LDS.
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

template <int KVDT, int HD, int REP, bool FUSED, int WPB>
__global__ __launch_bounds__(WPB * K2_WAVE) void attn_kernel(const AttnArgs a)
{
    using T = typename KVT<KVDT>::T;
    constexpr int EPC = KVT<KVDT>::EPC;
    constexpr int LPP = HD / EPC;                  // lanes per position
    constexpr int PPI = K2_WAVE / LPP;             // positions per wave slot
    constexpr int NL = EPC >= 16 ? 2 : 4;          // slots per wave per iteration
    constexpr int NT = WPB * K2_WAVE;              // threads per block
    static_assert(LPP >= 1 && LPP <= K2_WAVE, "head_dim / dtype");

    __shared__ float qs[REP][HD];
    __shared__ float newkv[2][HD];
    __shared__ float red_o[WPB][REP][HD];
    __shared__ float red_ml[WPB][REP][2];
    __shared__ float tmp4[WPB];

    const int g = blockIdx.y, s = blockIdx.x, S = gridDim.x;
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
    constexpr bool QREG = REP * EPC <= 32;
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
            a.out[(int64_t)(g * REP + h) * HD + d] = o / L;
        } else {
            a.part[(pbase + h) * HD + d] = o;
            if (d == 0) {
                a.part_ml[(pbase + h) * 2] = M;
                a.part_ml[(pbase + h) * 2 + 1] = L;
            }
        }
    }
}

// Combine the S split partials of every query head in split order (a fixed
// order: run-to-run deterministic): M = max_s m_s, L = sum_s l_s e^(m_s - M),
// out = sum_s o_s e^(m_s - M) / L.  Grid = n_kv blocks.  A separate launch: the
// kernel boundary makes every block's partials visible, with no
// cross-block synchronisation inside a kernel.
template <int HD, int REP>
__global__ __launch_bounds__(K2_BLOCK) void attn_combine_kernel(const AttnArgs a)
{
    __shared__ float f[K2_ATTN_MAX_SPLITS][REP];
    __shared__ float Mh[REP], Linv[REP];
    const int g = blockIdx.x, S = a.S, tid = threadIdx.x;
    const float *ml = a.part_ml + (int64_t)g * S * REP * 2;
    for (int t = tid; t < S * REP; t += K2_BLOCK) f[t / REP][t % REP] = ml[(int64_t)t * 2];
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
        for (int q = 0; q < S; ++q) L += f[q][tid] * ml[((int64_t)q * REP + tid) * 2 + 1];
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
            for (int i = 0; i < 8; ++i) v[i] = po[(int64_t)(q + i) * REP * HD];
#pragma unroll
            for (int i = 0; i < 8; ++i) o += f[q + i][h] * v[i];
        }
        for (; q < S; ++q) o += f[q][h] * po[(int64_t)q * REP * HD];
        a.out[(int64_t)(g * REP + h) * HD + d] = o * Linv[h];
    }
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

// ------------------------------------------------------------------ host --

int attn_splits(int n_kv, int len, int *chunk)
{
    int target = K2_ATTN_TARGET_BLOCKS / n_kv;
    if (target < 1) target = 1;
    int c = (len + target - 1) / target;
    if (c < K2_ATTN_MIN_CHUNK) c = K2_ATTN_MIN_CHUNK;
    if (c > K2_ATTN_MAX_CHUNK) c = K2_ATTN_MAX_CHUNK;
    *chunk = c;
    return (len + c - 1) / c;
}

static int attn_max_splits(int n_kv, int cap)
{
    int target = K2_ATTN_TARGET_BLOCKS / n_kv;
    if (target < 1) target = 1;
    const int by_chunk = (cap + K2_ATTN_MAX_CHUNK - 1) / K2_ATTN_MAX_CHUNK;
    return target > by_chunk ? target : by_chunk;
}

size_t attn_ws_bytes(int n_qh, int n_kv, int hd, int cap)
{
    const size_t S = (size_t)attn_max_splits(n_kv, cap);
    const size_t rep = (size_t)(n_qh / n_kv);
    return k2_align256((size_t)n_kv * S * rep * hd * 4) + k2_align256((size_t)n_kv * S * rep * 2 * 4);
}

void attn_ws_carve(void *ws, int n_qh, int n_kv, int hd, int cap, AttnArgs &a)
{
    const size_t S = (size_t)attn_max_splits(n_kv, cap);
    const size_t rep = (size_t)(n_qh / n_kv);
    char *p = (char *)ws;
    a.part = (float *)p;
    p += k2_align256((size_t)n_kv * S * rep * hd * 4);
    a.part_ml = (float *)p;
    p += k2_align256((size_t)n_kv * S * rep * 2 * 4);
}

template <int KVDT, int HD, int REP, bool FUSED>
static int attn_go(const AttnArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((attn_kernel<KVDT, HD, REP, FUSED, K2_WAVES_PER_BLOCK>), dim3(a.S, a.n_kv),
                       dim3(K2_BLOCK), 0, st, a);
    K2_CHECK_LAUNCH();
    if (a.S > 1) {
        hipLaunchKernelGGL((attn_combine_kernel<HD, REP>), dim3(a.n_kv), dim3(K2_BLOCK), 0, st, a);
        K2_CHECK_LAUNCH();
    }
    return K2_OK;
}

template <int KVDT, int HD, bool FUSED>
static int attn_rep(int rep, const AttnArgs &a, hipStream_t st)
{
    switch (rep) {
    case 1: return attn_go<KVDT, HD, 1, FUSED>(a, st);
    case 2: return attn_go<KVDT, HD, 2, FUSED>(a, st);
    case 4: return attn_go<KVDT, HD, 4, FUSED>(a, st);
    case 8: return attn_go<KVDT, HD, 8, FUSED>(a, st);
    }
    return K2_EUNSUPPORTED;
}

template <int KVDT, bool FUSED>
static int attn_hd(int hd, int rep, const AttnArgs &a, hipStream_t st)
{
    switch (hd) {
    case 16: return attn_rep<KVDT, 16, FUSED>(rep, a, st);
    case 32: return attn_rep<KVDT, 32, FUSED>(rep, a, st);
    case 64: return attn_rep<KVDT, 64, FUSED>(rep, a, st);
    case 128: return attn_rep<KVDT, 128, FUSED>(rep, a, st);
    }
    return K2_EUNSUPPORTED;
}

int attn_launch(int kvdt, int hd, int rep, bool fused, const AttnArgs &a, hipStream_t st)
{
    if (fused) {
        switch (kvdt) {
        case K2_F32: return attn_hd<K2_F32, true>(hd, rep, a, st);
        case K2_BF16: return attn_hd<K2_BF16, true>(hd, rep, a, st);
        case K2_I8: return attn_hd<K2_I8, true>(hd, rep, a, st);
        }
    } else {
        switch (kvdt) {
        case K2_F32: return attn_hd<K2_F32, false>(hd, rep, a, st);
        case K2_BF16: return attn_hd<K2_BF16, false>(hd, rep, a, st);
        case K2_I8: return attn_hd<K2_I8, false>(hd, rep, a, st);
        }
    }
    return K2_EUNSUPPORTED;
}

template <int KVDT>
static int kv_append_go(int hd, const float *k, const float *v, void *kc, void *vc, float *ks,
                        float *vs, int n_kv, int cap, int pos, hipStream_t st)
{
#define K2_APP(H)                                                                                  \
    case H:                                                                                        \
        hipLaunchKernelGGL((kv_append_kernel<KVDT, H>), dim3(n_kv), dim3(K2_BLOCK), 0, st, k, v, kc, \
                           vc, ks, vs, cap, pos);                                                  \
        break;
    switch (hd) {
        K2_APP(16)
        K2_APP(32)
        K2_APP(64)
        K2_APP(128)
    default: return K2_EUNSUPPORTED;
    }
#undef K2_APP
    K2_CHECK_LAUNCH();
    return K2_OK;
}

static bool hd_ok(int hd) { return hd == 16 || hd == 32 || hd == 64 || hd == 128; }
static bool rep_ok(int n_qh, int n_kv)
{
    if (n_kv <= 0 || n_qh <= 0 || n_qh % n_kv) return false;
    const int r = n_qh / n_kv;
    return r == 1 || r == 2 || r == 4 || r == 8;
}

}  // namespace k2

using namespace k2;

extern "C" size_t k2_attn_workspace_bytes(int n_qh, int n_kv, int head_dim, int cap)
{
    if (n_qh <= 0 || n_kv <= 0 || head_dim <= 0 || cap <= 0 || n_qh % n_kv) return 0;
    return attn_ws_bytes(n_qh, n_kv, head_dim, cap);
}

extern "C" int k2_kv_append(k2_dtype kvdt, const float *k, const float *v, void *kc, void *vc,
                            int n_kv, int head_dim, int cap, int pos, void *stream)
{
    if (!k2_ptr_ok(k) || !k2_ptr_ok(v) || !k2_ptr_ok(kc) || !k2_ptr_ok(vc)) return K2_EINVAL;
    if (n_kv <= 0 || cap <= 0) return K2_EINVAL;
    if (!hd_ok(head_dim)) return K2_EUNSUPPORTED;
    if (pos < 0 || pos >= cap) return K2_ERANGE;
    if (kvdt == K2_F32)
        return kv_append_go<K2_F32>(head_dim, k, v, kc, vc, nullptr, nullptr, n_kv, cap, pos, k2_stream(stream));
    if (kvdt == K2_BF16)
        return kv_append_go<K2_BF16>(head_dim, k, v, kc, vc, nullptr, nullptr, n_kv, cap, pos, k2_stream(stream));
    return K2_EUNSUPPORTED;
}

extern "C" int k2_kv_append_int8(const float *k, const float *v, int8_t *kc, int8_t *vc, float *ks,
                                 float *vs, int n_kv, int head_dim, int cap, int pos, void *stream)
{
    if (!k2_ptr_ok(k) || !k2_ptr_ok(v) || !k2_ptr_ok(kc) || !k2_ptr_ok(vc) || !k2_ptr_ok(ks) ||
        !k2_ptr_ok(vs))
        return K2_EINVAL;
    if (n_kv <= 0 || cap <= 0) return K2_EINVAL;
    if (!hd_ok(head_dim)) return K2_EUNSUPPORTED;
    if (pos < 0 || pos >= cap) return K2_ERANGE;
    return kv_append_go<K2_I8>(head_dim, k, v, kc, vc, ks, vs, n_kv, cap, pos, k2_stream(stream));
}

static int attn_common_check(k2_dtype kvdt, const void *kc, const void *vc, const float *ks,
                             const float *vs, const float *out, int n_qh, int n_kv, int head_dim,
                             int cap, void *ws, size_t ws_bytes)
{
    if (!k2_ptr_ok(kc) || !k2_ptr_ok(vc) || !k2_ptr_ok(out)) return K2_EINVAL;
    if (kvdt == K2_I8 && (!k2_ptr_ok(ks) || !k2_ptr_ok(vs))) return K2_EINVAL;
    if (n_qh <= 0 || n_kv <= 0 || cap <= 0) return K2_EINVAL;
    if (kvdt != K2_F32 && kvdt != K2_BF16 && kvdt != K2_I8) return K2_EUNSUPPORTED;
    if (!hd_ok(head_dim) || !rep_ok(n_qh, n_kv)) return K2_EUNSUPPORTED;
    if (cap > K2_ATTN_MAX_SPLITS * K2_ATTN_MAX_CHUNK) return K2_EUNSUPPORTED;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < attn_ws_bytes(n_qh, n_kv, head_dim, cap))
        return K2_EINVAL;
    return K2_OK;
}

extern "C" int k2_gqa_decode_attn(k2_dtype kvdt, const float *q, const void *kc, const void *vc,
                                  const float *ks, const float *vs, float *out, int n_qh, int n_kv,
                                  int head_dim, int cap, int len, float scale, void *ws,
                                  size_t ws_bytes, void *stream)
{
    int rc = attn_common_check(kvdt, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, ws, ws_bytes);
    if (rc) return rc;
    if (!k2_ptr_ok(q)) return K2_EINVAL;
    if (len < 1 || len > cap) return K2_ERANGE;
    AttnArgs a{};
    attn_ws_carve(ws, n_qh, n_kv, head_dim, cap, a);
    a.q = q;
    a.kc = const_cast<void *>(kc);
    a.vc = const_cast<void *>(vc);
    a.ks = const_cast<float *>(ks);
    a.vs = const_cast<float *>(vs);
    a.out = out;
    a.n_qh = n_qh;
    a.n_kv = n_kv;
    a.cap = cap;
    a.len = len;
    a.pos = len - 1;
    a.scale = scale;
    a.S = attn_splits(n_kv, len, &a.chunk);
    return attn_launch(kvdt, head_dim, n_qh / n_kv, false, a, k2_stream(stream));
}

extern "C" int k2_rope_append_attn(k2_dtype kvdt, const float *qkv, const float *cos_sin, void *kc,
                                   void *vc, float *ks, float *vs, float *out, int n_qh, int n_kv,
                                   int head_dim, int cap, int pos, void *ws, size_t ws_bytes,
                                   void *stream)
{
    int rc = attn_common_check(kvdt, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, ws, ws_bytes);
    if (rc) return rc;
    if (!k2_ptr_ok(qkv) || !k2_ptr_ok(cos_sin)) return K2_EINVAL;
    if (pos < 0 || pos >= cap) return K2_ERANGE;
    AttnArgs a{};
    attn_ws_carve(ws, n_qh, n_kv, head_dim, cap, a);
    a.qkv = qkv;
    a.cos_sin = cos_sin;
    a.kc = kc;
    a.vc = vc;
    a.ks = ks;
    a.vs = vs;
    a.out = out;
    a.n_qh = n_qh;
    a.n_kv = n_kv;
    a.cap = cap;
    a.pos = pos;
    a.len = pos + 1;
    a.scale = 1.0f / sqrtf((float)head_dim);
    a.S = attn_splits(n_kv, a.len, &a.chunk);
    return attn_launch(kvdt, head_dim, n_qh / n_kv, true, a, k2_stream(stream));
}
