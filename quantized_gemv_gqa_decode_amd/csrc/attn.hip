// attn.hip -- split-K GQA decode attention for gfx950, with the RoPE and
// KV-cache append of the new position fused in: launchers and C ABI (the
// device code is in attn_impl.h).
#include <atomic>

#include "attn_impl.h"

namespace k2 {

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

int attn_max_splits(int n_kv, int cap)
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
    return k2_align256((size_t)n_kv * S * rep * hd * 4) + k2_align256((size_t)n_kv * S * rep * 2 * 4) +
           k2_align256((size_t)n_kv * 4) + k2_align256((size_t)AO_SYNC_WORDS * 4);
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
    a.head_cnt = (unsigned *)p;
    p += k2_align256((size_t)n_kv * 4);
    a.ao_sync = (unsigned *)p;
}

// Compute units of the current device (cached per device id).
int device_cus()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int KVDT, int HD, int REP, bool FUSED>
static int attn_go(const AttnArgs &a, hipStream_t st)
{
    constexpr size_t lds = sizeof(float) * attn_stream_lds_floats<KVDT, HD, REP>();
    static_assert(lds <= 160 * 1024, "attention LDS per block");
    // Prefetch rows only fill compute units the attention blocks leave idle
    // (one block per compute unit at this LDS size).
    int rows = 0;
    if (a.pf && a.pf_bytes >= 16) {
        const int free_blocks = device_cus() - a.S * a.n_kv;
        rows = free_blocks > 0 ? free_blocks / a.S : 0;
    }
    hipLaunchKernelGGL((attn_kernel<KVDT, HD, REP, FUSED>), dim3(a.S, a.n_kv + rows), dim3(ATT_NT), lds, st,
                       a);
    K2_CHECK_LAUNCH();
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

// ------------------------------------------------ no-allocation variant --
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): k2_gqa_decode_attn with
// its workspace (split partials, their (max, sum) pairs and the per-kv-head
// arrival counters) in this file-scope device array instead of a caller
// buffer.  Each device holds its own copy until the process ends; its
// address comes from hipGetSymbolAddress on the first call on that device
// (in host code the array's name is not a device address).
constexpr size_t K2_SCRATCH_BYTES = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[K2_SCRATCH_BYTES];
static std::atomic<void *> g_scratch_dev[64];

// This device's address of `scratch` (set up once per device, with that
// device current), or nullptr on a runtime error.
static void *scratch_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void *p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        g_scratch_dev[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

__global__ void zero_u32_kernel(unsigned *p, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

extern "C" size_t k2_gqa_decode_attn_scratch_limit(void) { return K2_SCRATCH_BYTES; }

extern "C" int k2_gqa_decode_attn_noalloc(k2_dtype kvdt, const float *q, const void *kc, const void *vc,
                                          const float *ks, const float *vs, float *out, int n_qh,
                                          int n_kv, int head_dim, int cap, int len, float scale,
                                          void *stream)
{
    if (n_qh <= 0 || n_kv <= 0 || head_dim <= 0 || cap <= 0 || n_qh % n_kv) return K2_EINVAL;
    const size_t need = attn_ws_bytes(n_qh, n_kv, head_dim, cap);
    if (need > K2_SCRATCH_BYTES) return K2_EUNSUPPORTED;   // beyond the scratch array
    void *ws = scratch_ptr();
    if (!ws) return K2_EHIP;
    int rc = attn_common_check(kvdt, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, ws, need);
    if (rc) return rc;
    if (!k2_ptr_ok(q)) return K2_EINVAL;
    if (len < 1 || len > cap) return K2_ERANGE;
    AttnArgs a{};
    attn_ws_carve(ws, n_qh, n_kv, head_dim, cap, a);
    // the arrival counters must start at zero: the array keeps whatever the
    // last call on this device left (a fill kernel, not a memset node, so
    // that the call can sit inside a captured graph)
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, k2_stream(stream), a.head_cnt, n_kv);
    K2_CHECK_LAUNCH();
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

static int64_t weight_code_bytes(int wdt, int64_t N, int64_t K)
{
    switch (wdt) {
    case K2_F32: return N * K * 4;
    case K2_BF16: return N * K * 2;
    case K2_FP8E4M3: return N * K;
    default: return N * K / 2;
    }
}

int k2::attn_then_o(int wdt, int kvdt, int hd, int rep, AttnArgs at, const GemvArgs &o, int32_t *d_err,
                hipStream_t st)
{
    int rc;
    // int8 caches keep the two launches: measured at the 3.7B shape (int8
    // KV, ctx 4096) the one launch was 1.6 % (MXFP4) and 2.3 % (Q4S) slower
    // per decode step and even with fp8 weights, while with a bf16 cache it
    // is 1.8 % faster
    if (kvdt != K2_I8) {
        rc = attn_o_launch(wdt, kvdt, hd, rep, at, o, d_err, st);
        if (rc != K2_EUNSUPPORTED) return rc;
    }
    // the attention launch's idle compute units read the O weights once so
    // that they sit in the memory-side cache when the GEMV streams them
    at.pf = o.W;
    at.pf_bytes = weight_code_bytes(wdt, o.N, o.K);
    if ((rc = attn_launch(kvdt, hd, rep, true, at, st))) return rc;
    return gemv_dispatch(wdt, o, PRO_NONE, EPI_PLAIN, st);
}

extern "C" int k2_rope_append_attn_o(k2_dtype kvdt, const float *qkv, const float *cos_sin, void *kc,
                                     void *vc, float *ks, float *vs, float *out, int n_qh, int n_kv,
                                     int head_dim, int cap, int pos, k2_dtype wdt, const void *Wo,
                                     const void *Wo_s, float *h, int hidden, void *ws, size_t ws_bytes,
                                     int32_t *d_err, void *stream)
{
    int rc = attn_common_check(kvdt, kc, vc, ks, vs, out, n_qh, n_kv, head_dim, cap, ws, ws_bytes);
    if (rc) return rc;
    if (!k2_ptr_ok(qkv) || !k2_ptr_ok(cos_sin) || !k2_ptr_ok(Wo) || !k2_ptr_ok(h)) return K2_EINVAL;
    if ((wdt == K2_FP8E4M3 || wdt == K2_MXFP4 || wdt == K2_Q4S) && !k2_ptr_ok(Wo_s)) return K2_EINVAL;
    if (hidden <= 0) return K2_EINVAL;
    if (wdt != K2_F32 && wdt != K2_BF16 && wdt != K2_FP8E4M3 && wdt != K2_MXFP4 && wdt != K2_Q4S)
        return K2_EUNSUPPORTED;
    const int K = n_qh * head_dim;
    if (K % 32 || K > K2_MAX_LDS_FLOATS || (wdt == K2_Q4S && K % 64)) return K2_EUNSUPPORTED;
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
    GemvArgs o{};
    o.W = Wo;
    o.Sf = (const float *)Wo_s;
    o.S8 = (const uint8_t *)Wo_s;
    o.x = out;
    o.y = h;
    o.residual = h;
    o.N = hidden;
    o.K = K;
    o.B = 1;
    return attn_then_o(wdt, kvdt, head_dim, n_qh / n_kv, a, o, d_err, k2_stream(stream));
}

#ifdef K2_ATTN_TRACE
extern "C" int k2_attn_trace_read(unsigned long long *out, int n)
{
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(k2::k2_attn_trace), sizeof(unsigned long long) * n) ==
                   hipSuccess ? 0 : -4;
}
#endif
