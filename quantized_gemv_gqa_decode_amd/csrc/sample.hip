// sample.hip -- seeded sampling of the next token from the logits on the
// device ([k2-burn] "Project layout": sampling.rs, temperature / top-k /
// top-p / min-p / repetition penalty).
//
// Order of the filters (the conventional one; the pages name only the
// filters): repetition penalty on the distinct ids of `prev` (l > 0 -> l / r,
// else l * r), temperature, top-k (ties: lower id first), softmax, top-p
// (shortest prefix reaching top_p), min-p (p >= min_p * max p), then the
// first kept token whose cumulative probability exceeds u * the kept total.
// u = (first word of Philox4x32-10(counter, seed) >> 8) * 2^-24 (Salmon et
// al., SC 2011), the same 24-bit value everywhere.
//
// The penalty never raises a logit, so the top-k after it lies among the
// top kk = k + n_prev raw logits (kk <= 128).  Selection is a radix select,
// not a sort: logits map to order-preserving 32-bit keys, four passes pick the
// key of the kk-th largest one 8-bit digit at a time (a 256-bin LDS histogram
// and one wave's scan per pass), and a second select on the inverted ids
// breaks ties at that key in favour of lower ids.  Every 2048-wide slice keeps
// its kk best (one block each), a second round of the same kernel does the
// same over the survivors (at most 8 blocks), one block applies the penalty to
// what is left and selects the k best, and one wave sorts them in registers
// and does the rest with wave scans.
#include "k2_dev.h"

namespace k2 {

constexpr int SP_SLICE = 2048;             // logits per selection block
constexpr int SP_NT = 1024, SP_PER = SP_SLICE / SP_NT;
constexpr int SP_FINAL_NT = 1024, SP_FINAL_PER = 1;
constexpr int SP_MAX_SLICES = 128;         // vocab <= 262144: <= 128 * 128 survivors of the first round
constexpr int SP_MAX_K = 64, SP_MAX_PREV = 64, SP_MAX_KK = 128;
constexpr int SP_MAX_SLICES2 = SP_MAX_SLICES * SP_MAX_KK / SP_SLICE;   // second round: <= 8 blocks
static_assert(SP_MAX_SLICES2 * SP_MAX_KK <= SP_FINAL_NT * SP_FINAL_PER, "final block holds every candidate");

// a sorts before b: larger value, then lower id
__device__ __forceinline__ bool sp_before(float av, int ai, float bv, int bi)
{
    return av > bv || (av == bv && ai < bi);
}

// float -> unsigned key with the same order (-0 taken as +0); and back
__device__ __forceinline__ uint32_t sp_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float sp_val(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

struct SpLds {
    int hist[2][256];
    int digit[4], need[4], eq[4];
    int slot, dup;
};

// The need-th largest key among the live elements of the block (1 <= need <=
// their number), 8 bits per pass from the top.  On return n_above = how many
// live keys exceed it and n_eq how many equal it.  Expects s.hist[0] zeroed
// and visible; leaves it so.
template <int NT, int PER>
__device__ uint32_t sp_select(const uint32_t (&key)[PER], const bool (&live)[PER], int need, SpLds &s,
                              int &n_above, int &n_eq)
{
    const int want = need;
    uint32_t prefix = 0u, mask = 0u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int shift = 24 - 8 * p;
        int *h = s.hist[p & 1];
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (live[j] && (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> shift) & 255u], 1);
        for (int b = threadIdx.x; b < 256; b += NT) s.hist[(p + 1) & 1][b] = 0;
        __syncthreads();
        if (threadIdx.x < 64) {
            // lane l holds bins 255 - 4l .. 252 - 4l; an inclusive scan from the top bin
            const int lane = threadIdx.x, g0 = 255 - 4 * lane;
            const int c0 = h[g0], c1 = h[g0 - 1], c2 = h[g0 - 2], c3 = h[g0 - 3];
            const int tot = c0 + c1 + c2 + c3;
            int inc = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(inc, o, 64);
                if (lane >= o) inc += y;
            }
            const int exc = inc - tot;
            if (exc < need && need <= inc) {
                int above = exc, q, cq;
                if (above + c0 >= need) { q = 0; cq = c0; }
                else {
                    above += c0;
                    if (above + c1 >= need) { q = 1; cq = c1; }
                    else {
                        above += c1;
                        if (above + c2 >= need) { q = 2; cq = c2; }
                        else { above += c2; q = 3; cq = c3; }
                    }
                }
                s.digit[p] = g0 - q;
                s.need[p] = need - above;
                s.eq[p] = cq;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s.digit[p] << shift;
        mask |= 0xFFu << shift;
        need = s.need[p];
    }
    n_above = want - need;
    n_eq = s.eq[3];
    return prefix;
}

// take[j]: element j is one of the m best live elements (key desc, id asc);
// exactly m are taken over the block.  Expects s.dup == 0.
template <int NT, int PER>
__device__ void sp_top(const uint32_t (&key)[PER], const int (&id)[PER], const bool (&live)[PER], int m,
                       SpLds &s, bool (&take)[PER])
{
    int n_above, n_eq;
    const uint32_t t = sp_select<NT, PER>(key, live, m, s, n_above, n_eq);
    if (n_above + n_eq == m) {
#pragma unroll
        for (int j = 0; j < PER; ++j) take[j] = live[j] && key[j] >= t;
        return;
    }
    // more elements share key t than fit: the lowest ids among them
    uint32_t inv[PER];
    bool tied[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        inv[j] = ~(uint32_t)id[j];
        tied[j] = live[j] && key[j] == t;
    }
    int n2_above, n2_eq;
    const uint32_t t2 = sp_select<NT, PER>(inv, tied, m - n_above, s, n2_above, n2_eq);
    const int rest = m - n_above - n2_above;      // of the (duplicate) ids equal to ~t2
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        take[j] = live[j] && (key[j] > t || (tied[j] && inv[j] > t2));
        if (tied[j] && inv[j] == t2) take[j] = rest == n2_eq || atomicAdd(&s.dup, 1) < rest;
    }
}

// Selection: block b writes the kk best of entries [b * SP_SLICE, (b + 1) *
// SP_SLICE) of vin (ids: iin, or the position when iin is null) to cv/ci[b *
// kk, (b + 1) * kk), unordered (past n: -inf, id INT_MAX, after every real
// entry).
__global__ __launch_bounds__(SP_NT) void sample_sel_kernel(const float *vin, const int *iin, int n, int kk,
                                                           float *cv, int *ci)
{
    __shared__ SpLds s;
    const int base = blockIdx.x * SP_SLICE;
    uint32_t key[SP_PER];
    int id[SP_PER];
    bool live[SP_PER], take[SP_PER];
#pragma unroll
    for (int j = 0; j < SP_PER; ++j) {
        const int g = base + j * SP_NT + threadIdx.x;
        const bool ok = g < n;
        key[j] = ok ? sp_key(vin[g]) : 0u;
        id[j] = ok ? (iin ? iin[g] : g) : 0x7FFFFFFF;
        live[j] = true;
    }
    for (int b = threadIdx.x; b < 256; b += SP_NT) s.hist[0][b] = 0;
    if (threadIdx.x == 0) { s.slot = 0; s.dup = 0; }
    __syncthreads();
    sp_top<SP_NT, SP_PER>(key, id, live, kk, s, take);
#pragma unroll
    for (int j = 0; j < SP_PER; ++j) {
        if (!take[j]) continue;
        const int o = atomicAdd(&s.slot, 1);
        if (o >= kk) continue;                     // exactly kk are taken; the bound keeps writes in the slice
        cv[blockIdx.x * kk + o] = key[j] ? sp_val(key[j]) : -INFINITY;
        ci[blockIdx.x * kk + o] = id[j];
    }
}

// Philox4x32-10 of (counter, key): the first output word
__device__ __forceinline__ uint32_t philox_word0(uint64_t counter, uint64_t seed)
{
    uint32_t c0 = (uint32_t)counter, c1 = (uint32_t)(counter >> 32), c2 = 0u, c3 = 0u;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// a (value, id) pair's place in a 64-wide bitonic sort held by one wave, one
// element per lane: after the exchange with element i ^ j, the lower index of
// the pair holds the better of the two when its block of width w runs
// best-first, else the worse
__device__ __forceinline__ void sp_exchange(float &v, int &id, int i, int j, int w)
{
    const float pv = __shfl_xor(v, j, 64);
    const int pi = __shfl_xor(id, j, 64);
    const bool lower = (i & j) == 0, best_first = (i & w) == 0;
    // both lanes of the pair evaluate "the upper element beats the lower one"
    const bool upper_wins = lower ? sp_before(pv, pi, v, id) : sp_before(v, id, pv, pi);
    if (best_first ? upper_wins : !upper_wins) { v = pv; id = pi; }
}

// 64 (value, id) pairs, one per lane, best first
__device__ void sp_sort64(float &v, int &id)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int w = 2; w <= 64; w <<= 1) {
#pragma unroll
        for (int j = w >> 1; j > 0; j >>= 1) sp_exchange(v, id, lane, j, w);
    }
}

__device__ __forceinline__ float sp_scan(float x, int lane)      // inclusive prefix sum over the wave
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// One block: the n_cand candidates (which hold the k best after the
// penalty) penalised, the k best selected and sorted by one wave (k <= 64:
// lanes 0..k-1), then temperature, softmax, top-p, min-p and the draw.
__global__ __launch_bounds__(SP_FINAL_NT) void sample_final_kernel(const float *cv, const int *ci, int n_cand,
                                                                   int k, const k2_sampling sp,
                                                                   const int32_t *prev, int n_prev,
                                                                   uint64_t seed, uint64_t counter,
                                                                   int32_t *out)
{
    __shared__ SpLds s;
    __shared__ float tv[SP_MAX_K];
    __shared__ int ti[SP_MAX_K];
    __shared__ int pv[SP_MAX_PREV];
    constexpr int PER = SP_FINAL_PER;
    uint32_t key[PER];
    int id[PER];
    bool live[PER], take[PER];
    float val[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int g = j * SP_FINAL_NT + threadIdx.x;
        live[j] = g < n_cand;
        val[j] = live[j] ? cv[g] : -INFINITY;
        id[j] = live[j] ? ci[g] : 0x7FFFFFFF;
    }
    for (int b = threadIdx.x; b < 256; b += SP_FINAL_NT) s.hist[0][b] = 0;
    if (threadIdx.x < SP_MAX_K) { tv[threadIdx.x] = -INFINITY; ti[threadIdx.x] = 0x7FFFFFFF; }
    if (threadIdx.x < n_prev) pv[threadIdx.x] = prev[threadIdx.x];
    if (threadIdx.x == 0) { s.slot = 0; s.dup = 0; }
    __syncthreads();
    // repetition penalty, once per distinct id, then the k best
    const float rp = sp.repetition_penalty;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        bool seen = false;
#pragma unroll 8
        for (int p = 0; p < n_prev; ++p) seen |= pv[p] == id[j];
        if (seen && live[j]) val[j] = val[j] > 0.f ? val[j] / rp : val[j] * rp;
        key[j] = live[j] ? sp_key(val[j]) : 0u;
    }
    sp_top<SP_FINAL_NT, PER>(key, id, live, k, s, take);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (!take[j]) continue;
        const int o = atomicAdd(&s.slot, 1);
        if (o >= SP_MAX_K) continue;
        tv[o] = sp_val(key[j]);
        ti[o] = id[j];
    }
    __syncthreads();
    if (threadIdx.x >= 64) return;

    const int lane = threadIdx.x;
    float v0 = tv[lane];
    int i0 = ti[lane];
    sp_sort64(v0, i0);

    // lanes 0..k-1 now hold the top k, best first
    const bool in_k = lane < k;
    const float m = __shfl(v0, 0, 64) / sp.temperature;
    const float w = in_k ? expf(v0 / sp.temperature - m) : 0.f;
    const float sum = __shfl(sp_scan(w, lane), 63, 64);
    int n = k;
    if (sp.top_p < 1.f) {
        const float cum = sp_scan(w / sum, lane);
        const unsigned long long hit = __ballot(in_k && cum >= sp.top_p);
        if (hit) n = __ffsll((long long)hit);      // the shortest prefix reaching top_p
    }
    const float thr = sp.min_p * __shfl(w, 0, 64);
    const bool kept = lane < n && w >= thr;
    const float acc = sp_scan(kept ? w : 0.f, lane);
    const float total = __shfl(acc, 63, 64);
    const float u = (float)(philox_word0(counter, seed) >> 8) * 5.9604644775390625e-8f;   // 2^-24
    const unsigned long long over = __ballot(kept && acc > u * total);
    const unsigned long long all = __ballot(kept);
    const int at = over ? __ffsll((long long)over) - 1 : (all ? 63 - __clzll((long long)all) : 0);
    const int pick = __shfl(i0, at, 64);
    if (lane == 0) *out = pick;
}

}  // namespace k2

using namespace k2;

static int sp_slices(int n) { return (n + SP_SLICE - 1) / SP_SLICE; }

// per slice up to SP_MAX_KK (value, id) survivors: the first round's, then
// the second round's
static size_t sp_half_bytes(int vocab) { return k2_align256((size_t)sp_slices(vocab) * SP_MAX_KK * 4); }
static size_t sp_half2_bytes() { return k2_align256((size_t)SP_MAX_SLICES2 * SP_MAX_KK * 4); }

namespace k2 {
size_t sample_full_ws_bytes(int vocab);
int sample_full(const float *logits, int vocab, const k2_sampling &sp, const int32_t *prev, int n_prev,
                uint64_t seed, uint64_t counter, int32_t *out, void *ws, hipStream_t st);
}

constexpr int SP_MAX_VOCAB = 1 << 24;

extern "C" size_t k2_sample_workspace_bytes(int vocab)
{
    if (vocab <= 0 || vocab > SP_MAX_VOCAB) return 0;
    const size_t full = sample_full_ws_bytes(vocab);
    if (sp_slices(vocab) > SP_MAX_SLICES) return full;
    const size_t fast = 2 * sp_half_bytes(vocab) + 2 * sp_half2_bytes();
    return fast > full ? fast : full;
}

extern "C" int k2_sample(const float *logits, int vocab, const k2_sampling *sp, const int32_t *prev,
                         int n_prev, uint64_t seed, uint64_t counter, int32_t *out_token, void *ws,
                         size_t ws_bytes, void *stream)
{
    if (!k2_ptr_ok(logits) || !sp || !out_token || !ws || ((uintptr_t)ws & 255u)) return K2_EINVAL;
    if (vocab <= 0 || n_prev < 0 || (n_prev > 0 && !prev)) return K2_EINVAL;
    if (vocab > SP_MAX_VOCAB) return K2_EUNSUPPORTED;
    if (sp->top_k < 0) return K2_EINVAL;
    if (!(sp->temperature > 0.f) || !(sp->top_p > 0.f && sp->top_p <= 1.f) ||
        !(sp->min_p >= 0.f && sp->min_p < 1.f) || !(sp->repetition_penalty >= 1.f))
        return K2_EINVAL;
    if (ws_bytes < k2_sample_workspace_bytes(vocab)) return K2_EINVAL;
    hipStream_t st = k2_stream(stream);
    // the whole-vocabulary path: top-k off or wider than one wave sorts, or
    // more previous ids than the candidate bound k + n_prev <= 128 allows
    if (sp->top_k == 0 || sp->top_k > SP_MAX_K || n_prev > SP_MAX_PREV || sp_slices(vocab) > SP_MAX_SLICES)
        return sample_full(logits, vocab, *sp, prev, n_prev, seed, counter, out_token, ws, st);
    const int k = sp->top_k < vocab ? sp->top_k : vocab;
    const int kk = sp->top_k + n_prev < vocab ? sp->top_k + n_prev : vocab;
    char *w = (char *)ws;
    float *cv = (float *)w;
    int *ci = (int *)(w + sp_half_bytes(vocab));
    float *cv2 = (float *)(w + 2 * sp_half_bytes(vocab));
    int *ci2 = (int *)(w + 2 * sp_half_bytes(vocab) + sp_half2_bytes());
    const int slices = sp_slices(vocab), n1 = slices * kk;
    hipLaunchKernelGGL(sample_sel_kernel, dim3(slices), dim3(SP_NT), 0, st, logits, nullptr, vocab, kk, cv, ci);
    K2_CHECK_LAUNCH();
    // a second round over the survivors: at most SP_MAX_SLICES2 blocks
    const int slices2 = sp_slices(n1);
    hipLaunchKernelGGL(sample_sel_kernel, dim3(slices2), dim3(SP_NT), 0, st, cv, ci, n1, kk, cv2, ci2);
    K2_CHECK_LAUNCH();
    hipLaunchKernelGGL(sample_final_kernel, dim3(1), dim3(SP_FINAL_NT), 0, st, cv2, ci2, slices2 * kk, k, *sp,
                       prev, n_prev, seed, counter, out_token);
    K2_CHECK_LAUNCH();
    return K2_OK;
}
