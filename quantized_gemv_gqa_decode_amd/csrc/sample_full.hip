// sample_full.hip -- seeded sampling over the WHOLE vocabulary ([k2-burn]
// "Usage": --top-k / --top-p / --min-p as separate truncation filters,
// --repetition-penalty on already-seen tokens): top-k off (0) or above the
// 64 that the one-wave path of sample.hip sorts, and any number of
// previous ids.  Same filters, order and draw as sample.hip.
//
// Nothing is sorted.  Every decision is a selection in the order (z desc,
// id asc) by a running weight -- a count for top-k, the probability mass for
// top-p and the draw -- found by radix selection on order-preserving 32-bit
// keys of z, one 8-bit digit per launch from the top: every block histograms
// its slice of the candidates whose key matches the digits chosen so far
// (weights summed per bin), and the next launch's blocks each re-derive the
// chosen digits from the finished histograms.  A weight is an integer: the
// mass exp(z - m) in [0, 1] (fp32, m = the largest z) as a multiple of
// 2^-40, so bin sums are exact whatever order the blocks add them in, and
// the whole draw is run-to-run deterministic.  After the four digits the
// key T of the deciding element is known together with the weight above it;
// as every token with key T has the same weight, the number n of them
// needed is arithmetic, and the n-th lowest id among them is the least id
// of the bin (tracked per bin) when n = 1, or else found by one block
// scanning the vocabulary in id order.
//
// Launches: clear, previous-id bitmap, keys; then per active selection
// (top-k if 0 < k < vocab, top-p if top_p < 1, the draw) four digit rounds
// and one resolving block.
#include "k2_dev.h"

namespace k2 {

constexpr int SF_NT = 1024;
constexpr int SF_PER = 4;
constexpr int SF_SLICE = SF_NT * SF_PER;   // tokens per block
constexpr int SF_SELS = 3;                 // top-k, top-p, draw
constexpr int SF_BINS = 256;
constexpr double SF_SCALE = 1099511627776.0;   // 2^40

__device__ __forceinline__ uint32_t sf_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float sf_val(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// the state that later launches read (written by the resolving blocks)
struct SfState {
    uint32_t maxkey;           // key of the largest z
    uint32_t cutT[2];          // top-k, top-p: kept iff key > cutT, or key == cutT and id <= cutId
    int32_t cutId[2];
};

struct SfArgs {
    const float *logits;
    int vocab;
    float temperature, top_p, min_p, penalty;
    int top_k;
    int active;                // bit s: selection s runs
    const int32_t *prev;
    int n_prev;
    uint32_t *bits;            // [ceil(vocab / 32)]
    uint32_t *keys;            // [vocab]
    SfState *st;
    unsigned long long *hist;  // [SF_SELS * 4][256] weights
    uint32_t *cnt;             // [SF_SELS * 4][256] tokens
    uint32_t *minid;           // [SF_SELS * 4][256] least id
    uint64_t seed, counter;
    int32_t *out;
};

__device__ __forceinline__ unsigned long long sf_mass(float w)
{
    return (unsigned long long)__double2ull_rn((double)w * SF_SCALE);
}

// penalised, tempered logit of token i (sample.hip's arithmetic)
__device__ __forceinline__ float sf_z(const SfArgs &a, int i)
{
    float v = a.logits[i];
    if ((a.bits[i >> 5] >> (i & 31)) & 1u) v = v > 0.f ? v / a.penalty : v * a.penalty;
    return v / a.temperature;
}

// is token (key, id) a candidate of selection s, given the earlier ones
__device__ __forceinline__ bool sf_cand(const SfArgs &a, const SfState &st, int s, uint32_t key, int id,
                                        float m)
{
    if (s >= 1 && (a.active & 1)) {
        if (!(key > st.cutT[0] || (key == st.cutT[0] && id <= st.cutId[0]))) return false;
    }
    if (s >= 2) {
        if ((a.active & 2) && !(key > st.cutT[1] || (key == st.cutT[1] && id <= st.cutId[1]))) return false;
        if (a.min_p > 0.f && !(expf(sf_val(key) - m) >= a.min_p)) return false;
    }
    return true;
}

__device__ __forceinline__ unsigned long long sf_weight(int s, uint32_t key, float m)
{
    return s == 0 ? 1ull : sf_mass(expf(sf_val(key) - m));
}

// The selection's target weight once its first round is complete: top-k the
// count k; top-p the least integer >= top_p * total (at least 1); the draw
// floor(u * total) + 1 with u = word0 >> 8 over 2^24 (first cumulative above
// u * total).
__device__ unsigned long long sf_target(const SfArgs &a, int s, unsigned long long total)
{
    if (s == 0) return (unsigned long long)a.top_k;
    if (s == 1) {
        unsigned long long t = (unsigned long long)ceil((double)a.top_p * (double)total);
        return t < 1ull ? 1ull : (t > total ? total : t);
    }
    uint32_t c0 = (uint32_t)a.counter, c1 = (uint32_t)(a.counter >> 32), c2 = 0u, c3 = 0u;
    uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    for (int r = 0; r < 10; ++r) {             // Philox4x32-10, as sample.hip
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    const unsigned long long u24 = c0 >> 8;
    const unsigned long long lo = u24 * total, hi = __umul64hi(u24, total);
    return ((hi << 40) | (lo >> 24)) + 1ull;   // floor(u24 * total / 2^24) + 1
}

// Digits 0 .. r-1 of selection s re-derived from its finished histograms
// (wave 0; the result in every thread through LDS): prefix/mask of the key,
// the weight of the candidates above that prefix region, the target.
struct SfWalk {
    uint32_t prefix, mask;
    unsigned long long above, target;
    int digit;                 // the last digit chosen
};

__device__ void sf_walk(const SfArgs &a, int s, int r, SfWalk &w)
{
    __shared__ SfWalk sw;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint32_t prefix = 0u, mask = 0u;
        unsigned long long above = 0ull, target = 0ull;
        int digit = 0;
        for (int q = 0; q < r; ++q) {
            const unsigned long long *h = a.hist + (size_t)(4 * s + q) * SF_BINS;
            // lane l holds bins 255 - 4l .. 252 - 4l; inclusive sums from the top bin
            const int g0 = 255 - 4 * lane;
            const unsigned long long b0 = h[g0], b1 = h[g0 - 1], b2 = h[g0 - 2], b3 = h[g0 - 3];
            const unsigned long long tot = b0 + b1 + b2 + b3;
            unsigned long long inc = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const unsigned long long y = __shfl_up(inc, o, 64);
                if (lane >= o) inc += y;
            }
            if (q == 0) target = sf_target(a, s, __shfl(inc, 63, 64));
            const unsigned long long exc = inc - tot;
            const unsigned long long need = target - above;    // >= 1
            const bool here = exc < need && need <= inc;
            const unsigned long long hit = __ballot(here);
            const int src = __ffsll((long long)hit) - 1;       // exactly one lane (need <= the total)
            int d = 0;
            unsigned long long ab = 0ull;
            if (here) {
                unsigned long long acc = exc;
                if (acc + b0 >= need) d = g0;
                else {
                    acc += b0;
                    if (acc + b1 >= need) d = g0 - 1;
                    else {
                        acc += b1;
                        if (acc + b2 >= need) d = g0 - 2;
                        else { acc += b2; d = g0 - 3; }
                    }
                }
                ab = acc;
            }
            d = __shfl(d, src < 0 ? 0 : src, 64);
            ab = __shfl(ab, src < 0 ? 0 : src, 64);
            above += ab;
            const int shift = 24 - 8 * q;
            prefix |= (uint32_t)d << shift;
            mask |= 0xFFu << shift;
            digit = d;
        }
        if (lane == 0) {
            sw.prefix = prefix;
            sw.mask = mask;
            sw.above = above;
            sw.target = target;
            sw.digit = digit;
        }
    }
    __syncthreads();
    w = sw;
}

__global__ void sf_clear_kernel(SfArgs a)
{
    const int nb = (a.vocab + 31) >> 5;
    const int nh = SF_SELS * 4 * SF_BINS;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nh + nb; i += gridDim.x * blockDim.x) {
        if (i < nh) {
            a.hist[i] = 0ull;
            a.cnt[i] = 0u;
            a.minid[i] = 0xFFFFFFFFu;
        } else {
            a.bits[i - nh] = 0u;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.st->maxkey = 0u;
        a.st->cutT[0] = a.st->cutT[1] = 0u;
        a.st->cutId[0] = a.st->cutId[1] = 0x7FFFFFFF;
    }
}

__global__ void sf_bits_kernel(SfArgs a)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < a.n_prev) {
        const int t = a.prev[i];
        if (t >= 0 && t < a.vocab) atomicOr(&a.bits[t >> 5], 1u << (t & 31));
    }
}

__global__ __launch_bounds__(SF_NT) void sf_keys_kernel(SfArgs a)
{
    __shared__ uint32_t bm[SF_NT / 64];
    uint32_t best = 0u;
#pragma unroll
    for (int j = 0; j < SF_PER; ++j) {
        const int i = blockIdx.x * SF_SLICE + j * SF_NT + threadIdx.x;
        if (i < a.vocab) {
            const uint32_t k = sf_key(sf_z(a, i));
            a.keys[i] = k;
            best = k > best ? k : best;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t y = __shfl_xor(best, o, 64);
        best = y > best ? y : best;
    }
    if ((threadIdx.x & 63) == 0) bm[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < SF_NT / 64; ++w) best = bm[w] > best ? bm[w] : best;
        atomicMax(&a.st->maxkey, best);
    }
}

// digit r of selection s over this block's slice
__global__ __launch_bounds__(SF_NT) void sf_round_kernel(SfArgs a, int s, int r)
{
    __shared__ unsigned long long lw[SF_BINS];
    __shared__ uint32_t lc[SF_BINS], lm[SF_BINS];
    for (int b = threadIdx.x; b < SF_BINS; b += SF_NT) { lw[b] = 0ull; lc[b] = 0u; lm[b] = 0xFFFFFFFFu; }
    SfWalk w;
    sf_walk(a, s, r, w);                          // its barrier also orders the LDS clears
    const SfState st = *a.st;
    const float m = sf_val(st.maxkey);
    const int shift = 24 - 8 * r;
#pragma unroll
    for (int j = 0; j < SF_PER; ++j) {
        const int i = blockIdx.x * SF_SLICE + j * SF_NT + threadIdx.x;
        if (i >= a.vocab) continue;
        const uint32_t key = a.keys[i];
        if ((key & w.mask) != w.prefix || !sf_cand(a, st, s, key, i, m)) continue;
        const int d = (key >> shift) & 255;
        atomicAdd(&lw[d], sf_weight(s, key, m));
        atomicAdd(&lc[d], 1u);
        if (r == 3) atomicMin(&lm[d], (uint32_t)i);
    }
    __syncthreads();
    const size_t base = (size_t)(4 * s + r) * SF_BINS;
    for (int b = threadIdx.x; b < SF_BINS; b += SF_NT) {
        if (lc[b]) {
            atomicAdd(&a.hist[base + b], lw[b]);
            atomicAdd(&a.cnt[base + b], lc[b]);
            if (r == 3) atomicMin(&a.minid[base + b], lm[b]);
        }
    }
}

// One block: the key T of selection s's deciding element, how many of the
// tokens with key T it takes (n), and the n-th lowest id among them: the
// bin's least id when n = 1, all of them when n is their count (top-k,
// top-p), else a scan of the vocabulary in id order.  Top-k / top-p store
// the cut; the draw stores the token.
__global__ __launch_bounds__(SF_NT) void sf_resolve_kernel(SfArgs a, int s)
{
    __shared__ int cut_s;
    __shared__ uint32_t tally[SF_NT];
    SfWalk w;
    sf_walk(a, s, 4, w);
    const uint32_t T = w.prefix;
    const SfState st = *a.st;
    const float m = sf_val(st.maxkey);
    const size_t bin = (size_t)(4 * s + 3) * SF_BINS + w.digit;
    const uint32_t n_tie = a.cnt[bin];
    const unsigned long long wt = sf_weight(s, T, m);
    const unsigned long long need = w.target - w.above;                // >= 1
    uint32_t n = (uint32_t)((need + wt - 1) / (wt ? wt : 1ull));
    n = n < 1u ? 1u : (n > n_tie ? n_tie : n);
    int cut;
    if (n == 1u) cut = (int)a.minid[bin];
    else if (n == n_tie && s < 2) cut = 0x7FFFFFFF;
    else {
        // the n-th candidate with key T in id order: each thread counts its
        // contiguous range, an exclusive scan finds the range holding it
        const int per = (a.vocab + SF_NT - 1) / SF_NT;
        const int lo = threadIdx.x * per, hi = lo + per < a.vocab ? lo + per : a.vocab;
        uint32_t c = 0u;
        for (int i = lo; i < hi; ++i) c += a.keys[i] == T && sf_cand(a, st, s, T, i, m);
        tally[threadIdx.x] = c;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t acc = 0u;
            for (int t = 0; t < SF_NT; ++t) { const uint32_t v = tally[t]; tally[t] = acc; acc += v; }
        }
        __syncthreads();
        if (threadIdx.x == 0) cut_s = 0x7FFFFFFF;
        __syncthreads();
        uint32_t seen = tally[threadIdx.x];
        if (seen < n && seen + c >= n) {
            for (int i = lo; i < hi; ++i) {
                if (a.keys[i] == T && sf_cand(a, st, s, T, i, m) && ++seen == n) { cut_s = i; break; }
            }
        }
        __syncthreads();
        cut = cut_s;
    }
    if (threadIdx.x == 0) {
        if (s < 2) {
            a.st->cutT[s] = T;
            a.st->cutId[s] = cut;
        } else {
            *a.out = cut;
        }
    }
}

size_t sample_full_ws_bytes(int vocab)
{
    return k2_align256(sizeof(SfState)) + k2_align256((size_t)SF_SELS * 4 * SF_BINS * 8) +
           2 * k2_align256((size_t)SF_SELS * 4 * SF_BINS * 4) + k2_align256((size_t)((vocab + 31) / 32) * 4) +
           k2_align256((size_t)vocab * 4);
}

int sample_full(const float *logits, int vocab, const k2_sampling &sp, const int32_t *prev, int n_prev,
                uint64_t seed, uint64_t counter, int32_t *out, void *ws, hipStream_t st)
{
    SfArgs a{};
    char *p = (char *)ws;
    a.st = (SfState *)p;
    p += k2_align256(sizeof(SfState));
    a.hist = (unsigned long long *)p;
    p += k2_align256((size_t)SF_SELS * 4 * SF_BINS * 8);
    a.cnt = (uint32_t *)p;
    p += k2_align256((size_t)SF_SELS * 4 * SF_BINS * 4);
    a.minid = (uint32_t *)p;
    p += k2_align256((size_t)SF_SELS * 4 * SF_BINS * 4);
    a.bits = (uint32_t *)p;
    p += k2_align256((size_t)((vocab + 31) / 32) * 4);
    a.keys = (uint32_t *)p;
    a.logits = logits;
    a.vocab = vocab;
    a.temperature = sp.temperature;
    a.top_p = sp.top_p;
    a.min_p = sp.min_p;
    a.penalty = sp.repetition_penalty;
    a.top_k = sp.top_k;
    a.active = (sp.top_k > 0 && sp.top_k < vocab ? 1 : 0) | (sp.top_p < 1.f ? 2 : 0) | 4;
    a.prev = prev;
    a.n_prev = n_prev;
    a.seed = seed;
    a.counter = counter;
    a.out = out;
    const int slices = (vocab + SF_SLICE - 1) / SF_SLICE;
    hipLaunchKernelGGL(sf_clear_kernel, dim3(16), dim3(256), 0, st, a);
    K2_CHECK_LAUNCH();
    if (n_prev > 0) {
        hipLaunchKernelGGL(sf_bits_kernel, dim3((n_prev + 255) / 256), dim3(256), 0, st, a);
        K2_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(sf_keys_kernel, dim3(slices), dim3(SF_NT), 0, st, a);
    K2_CHECK_LAUNCH();
    for (int s = 0; s < SF_SELS; ++s) {
        if (!(a.active >> s & 1)) continue;
        for (int r = 0; r < 4; ++r) {
            hipLaunchKernelGGL(sf_round_kernel, dim3(slices), dim3(SF_NT), 0, st, a, s, r);
            K2_CHECK_LAUNCH();
        }
        hipLaunchKernelGGL(sf_resolve_kernel, dim3(1), dim3(SF_NT), 0, st, a, s);
        K2_CHECK_LAUNCH();
    }
    return K2_OK;
}

}  // namespace k2
