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
// top k + n_prev raw logits: a selection round keeps the best 128 of every
// 2048-wide slice (bitonic sort in LDS); two rounds leave at most 2048
// survivors, which one block sorts before doing the rest on at most 128
// candidates.
#include "k2_dev.h"

namespace k2 {

constexpr int SP_SLICE = 2048;             // values per selection block
constexpr int SP_KEEP = 128;               // survivors per slice (>= top_k + n_prev)
constexpr int SP_NT = 1024;
constexpr int SP_FINAL_NT = 1024;
constexpr int SP_MAX_SLICES = 128;         // vocab <= 262144: two selection rounds leave <= 2048
constexpr int SP_MAX_K = 64, SP_MAX_PREV = 64;

// a sorts before b: larger value, then lower id
__device__ __forceinline__ bool sp_before(float av, int ai, float bv, int bi)
{
    return av > bv || (av == bv && ai < bi);
}

// Bitonic sort of n (a power of two) (value, id) pairs in LDS, best first.
__device__ void sp_bitonic(float *v, int *id, int n)
{
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += blockDim.x) {
                const int l = i ^ j;
                if (l > i) {
                    const bool first = (i & k) == 0;
                    const bool sw = first ? sp_before(v[l], id[l], v[i], id[i])
                                          : sp_before(v[i], id[i], v[l], id[l]);
                    if (sw) {
                        const float tv = v[i]; v[i] = v[l]; v[l] = tv;
                        const int ti = id[i]; id[i] = id[l]; id[l] = ti;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// One selection round: block b keeps the best SP_KEEP of values
// [b * SP_SLICE, (b + 1) * SP_SLICE) of vin (ids: iin, or the position when
// iin is null).
__global__ __launch_bounds__(SP_NT) void sample_cand_kernel(const float *vin, const int *iin, int n, float *cv,
                                                            int *ci)
{
    __shared__ float v[SP_SLICE];
    __shared__ int id[SP_SLICE];
    const int base = blockIdx.x * SP_SLICE;
    for (int j = threadIdx.x; j < SP_SLICE; j += SP_NT) {
        const int g = base + j;
        const bool ok = g < n;
        v[j] = ok ? vin[g] : -INFINITY;
        id[j] = ok ? (iin ? iin[g] : g) : 0x7FFFFFFF;
    }
    __syncthreads();
    sp_bitonic(v, id, SP_SLICE);
    for (int j = threadIdx.x; j < SP_KEEP; j += SP_NT) {
        cv[blockIdx.x * SP_KEEP + j] = v[j];
        ci[blockIdx.x * SP_KEEP + j] = id[j];
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

__global__ __launch_bounds__(SP_FINAL_NT) void sample_final_kernel(const float *cv, const int *ci, int n_cand,
                                                                   int n_pow2, const k2_sampling sp,
                                                                   const int32_t *prev, int n_prev,
                                                                   uint64_t seed, uint64_t counter,
                                                                   int32_t *out)
{
    extern __shared__ float lds_f[];
    float *v = lds_f;
    int *id = reinterpret_cast<int *>(lds_f + n_pow2);
    __shared__ int pv[SP_MAX_PREV];
    for (int j = threadIdx.x; j < n_pow2; j += SP_FINAL_NT) {
        const bool ok = j < n_cand;
        v[j] = ok ? cv[j] : -INFINITY;
        id[j] = ok ? ci[j] : 0x7FFFFFFF;
    }
    for (int j = threadIdx.x; j < n_prev; j += SP_FINAL_NT) pv[j] = prev[j];
    __syncthreads();
    sp_bitonic(v, id, n_pow2);
    if (threadIdx.x != 0) return;

    // the top k + n_prev raw logits, penalised, re-sorted (insertion sort)
    const int kk = sp.top_k + n_prev < n_cand ? sp.top_k + n_prev : n_cand;
    for (int c = 0; c < kk; ++c) {
        bool seen = false;
        for (int p = 0; p < n_prev; ++p) seen |= pv[p] == id[c];
        if (seen) v[c] = v[c] > 0.f ? v[c] / sp.repetition_penalty : v[c] * sp.repetition_penalty;
    }
    for (int c = 1; c < kk; ++c) {
        const float tv = v[c];
        const int ti = id[c];
        int d = c - 1;
        while (d >= 0 && sp_before(tv, ti, v[d], id[d])) {
            v[d + 1] = v[d];
            id[d + 1] = id[d];
            --d;
        }
        v[d + 1] = tv;
        id[d + 1] = ti;
    }
    const int k = sp.top_k < kk ? sp.top_k : kk;
    // softmax over the top k (unnormalised weights in v), top-p, min-p
    const float m = v[0] / sp.temperature;
    float sum = 0.f;
    for (int c = 0; c < k; ++c) {
        v[c] = expf(v[c] / sp.temperature - m);
        sum += v[c];
    }
    int n = k;
    if (sp.top_p < 1.f) {
        float cum = 0.f;
        for (int c = 0; c < k; ++c) {
            cum += v[c] / sum;
            if (cum >= sp.top_p) { n = c + 1; break; }
        }
    }
    const float thr = sp.min_p * v[0];
    float total = 0.f;
    for (int c = 0; c < n; ++c) total += v[c] >= thr ? v[c] : 0.f;
    const float u = (float)(philox_word0(counter, seed) >> 8) * 5.9604644775390625e-8f;   // 2^-24
    const float target = u * total;
    float acc = 0.f;
    int pick = id[0];
    for (int c = 0; c < n; ++c) {
        if (v[c] < thr) continue;
        pick = id[c];
        acc += v[c];
        if (acc > target) break;
    }
    *out = pick;
}

}  // namespace k2

using namespace k2;

static int sp_slices(int n) { return (n + SP_SLICE - 1) / SP_SLICE; }

// two rounds of (values, ids) buffers: round 1 holds sp_slices(vocab) *
// SP_KEEP survivors, round 2 those of round 1's
static size_t sp_round_bytes(int n) { return k2_align256((size_t)sp_slices(n) * SP_KEEP * 4); }

extern "C" size_t k2_sample_workspace_bytes(int vocab)
{
    if (vocab <= 0 || sp_slices(vocab) > SP_MAX_SLICES) return 0;
    return 2 * sp_round_bytes(vocab) + 2 * sp_round_bytes(sp_slices(vocab) * SP_KEEP);
}

extern "C" int k2_sample(const float *logits, int vocab, const k2_sampling *sp, const int32_t *prev,
                         int n_prev, uint64_t seed, uint64_t counter, int32_t *out_token, void *ws,
                         size_t ws_bytes, void *stream)
{
    if (!k2_ptr_ok(logits) || !sp || !out_token || !ws || ((uintptr_t)ws & 255u)) return K2_EINVAL;
    if (vocab <= 0 || n_prev < 0 || (n_prev > 0 && !prev)) return K2_EINVAL;
    if (sp_slices(vocab) > SP_MAX_SLICES || n_prev > SP_MAX_PREV) return K2_EUNSUPPORTED;
    if (sp->top_k < 1 || sp->top_k > SP_MAX_K) return K2_EUNSUPPORTED;
    if (!(sp->temperature > 0.f) || !(sp->top_p > 0.f && sp->top_p <= 1.f) ||
        !(sp->min_p >= 0.f && sp->min_p < 1.f) || !(sp->repetition_penalty >= 1.f))
        return K2_EINVAL;
    if (ws_bytes < k2_sample_workspace_bytes(vocab)) return K2_EINVAL;
    hipStream_t st = k2_stream(stream);
    char *w = (char *)ws;
    float *cv = (float *)w;
    int *ci = (int *)(w + sp_round_bytes(vocab));
    hipLaunchKernelGGL(sample_cand_kernel, dim3(sp_slices(vocab)), dim3(SP_NT), 0, st, logits, nullptr, vocab, cv,
                       ci);
    K2_CHECK_LAUNCH();
    int n_cand = sp_slices(vocab) * SP_KEEP;
    if (n_cand > SP_SLICE) {                       // a second round over the survivors
        float *cv2 = (float *)(w + 2 * sp_round_bytes(vocab));
        int *ci2 = (int *)(w + 2 * sp_round_bytes(vocab) + sp_round_bytes(n_cand));
        hipLaunchKernelGGL(sample_cand_kernel, dim3(sp_slices(n_cand)), dim3(SP_NT), 0, st, cv, ci, n_cand, cv2,
                           ci2);
        K2_CHECK_LAUNCH();
        n_cand = sp_slices(n_cand) * SP_KEEP;
        cv = cv2;
        ci = ci2;
    }
    int n_pow2 = SP_KEEP;
    while (n_pow2 < n_cand) n_pow2 <<= 1;
    hipLaunchKernelGGL(sample_final_kernel, dim3(1), dim3(SP_FINAL_NT), (size_t)n_pow2 * 8, st, cv, ci, n_cand,
                       n_pow2, *sp, prev, n_prev, seed, counter, out_token);
    K2_CHECK_LAUNCH();
    return K2_OK;
}
