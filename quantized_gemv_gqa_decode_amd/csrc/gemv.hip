// gemv.hip -- weight-streaming dequantizing GEMV for gfx950.
//
// y = W_hat x for the projections of the decode step ([k2-burn] "Model
// shape": QKV, O, SwiGLU gate/up, down, untied lm_head) with W stored as
// fp32, bf16, fp8 E4M3FN + per-row scale ([k2-burn] "Quantization") or MXFP4
// (E2M1 + E8M0 per 32 columns; [k3_run.c] header comment).
//
// Layout of the work:
//   * A 256-thread block stages the B activation vectors in LDS once
//     (optionally applying the grouped RMSNorm on the way in), then its four
//     waves stream rows.
//   * A wave owns R rows at a time (a "unit").  Lane l reads 16-byte chunk
//     c = l, l+64, ... of each of the R rows, so every load instruction of
//     the wave covers 1 KiB of contiguous weights, and the activation chunk
//     read from LDS is reused by the R rows.  U chunks per row are loaded
//     before any arithmetic so that R*U loads (R*U KiB per wave) are in
//     flight.
//   * Rows are reduced across the wave with butterfly shuffles; the epilogue
//     writes y (plus residual), or silu(gate) * up for row pairs, or a
//     (max, index) candidate for the argmax that follows the lm_head.
//   * Units are distributed grid-stride so the grid can be capped while
//     every unit is still covered.
// A 16-byte chunk holds 4 fp32, 8 bf16, 16 fp8 or 32 E2M1 values; for MXFP4
// a chunk is exactly one 32-column scale block, so the E8M0 scale is applied
// once to each chunk's partial sum.
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

int gemv_dispatch_f32(const GemvArgs &a, int pro, int epi, hipStream_t st);
int gemv_dispatch_bf16(const GemvArgs &a, int pro, int epi, hipStream_t st);
int gemv_dispatch_fp8(const GemvArgs &a, int pro, int epi, hipStream_t st);
int gemv_dispatch_mxfp4(const GemvArgs &a, int pro, int epi, hipStream_t st);
int gemv_dispatch_q4s(const GemvArgs &a, int pro, int epi, hipStream_t st);

int gemv_dispatch(int wdt, const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    // a quantized format without its scales is refused here, not read at address 0
    if (((wdt == K2_FP8E4M3 || wdt == K2_Q4S) && !a.Sf) || (wdt == K2_MXFP4 && !a.S8)) return K2_EINVAL;
    switch (wdt) {
    case K2_F32: return gemv_dispatch_f32(a, pro, epi, st);
    case K2_BF16: return gemv_dispatch_bf16(a, pro, epi, st);
    case K2_FP8E4M3: return gemv_dispatch_fp8(a, pro, epi, st);
    case K2_MXFP4: return gemv_dispatch_mxfp4(a, pro, epi, st);
    case K2_Q4S: return gemv_dispatch_q4s(a, pro, epi, st);
    default: return K2_EUNSUPPORTED;
    }
}

}  // namespace k2


using namespace k2;

// Generic entry points: B vectors (1, 2, 4 or 8; 3, 5..7 are padded by the
// caller-visible rule below), no prologue, optional residual.
static int gemv_entry(int wdt, const void *W, const void *S, const float *x, float *y,
                      const float *residual, int N, int K, int B, void *stream)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(x) || !k2_ptr_ok(y)) return K2_EINVAL;
    if (residual && !k2_aligned16(residual)) return K2_EINVAL;
    if (N <= 0 || K <= 0 || B <= 0) return K2_EINVAL;
    if ((wdt == K2_FP8E4M3 || wdt == K2_MXFP4 || wdt == K2_Q4S) && !S) return K2_EINVAL;
    if (K % 32 != 0 || (int64_t)B * K > K2_MAX_LDS_FLOATS) return K2_EUNSUPPORTED;
    if (wdt == K2_Q4S && K % 64) return K2_EUNSUPPORTED;
    if (B != 1 && B != 2 && B != 4 && B != 8) return K2_EUNSUPPORTED;
    GemvArgs a{};
    a.W = W;
    a.Sf = (const float *)S;
    a.S8 = (const uint8_t *)S;
    a.x = x;
    a.y = y;
    a.residual = residual;
    a.N = N;
    a.K = K;
    a.B = B;
    return gemv_dispatch(wdt, a, PRO_NONE, EPI_PLAIN, k2_stream(stream));
}

extern "C" int k2_gemv_qbf16(const uint16_t *W, const float *x, float *y, const float *residual,
                             int N, int K, int B, void *stream)
{
    return gemv_entry(K2_BF16, W, nullptr, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_qfp8(const uint8_t *W, const float *row_scale, const float *x, float *y,
                            const float *residual, int N, int K, int B, void *stream)
{
    return gemv_entry(K2_FP8E4M3, W, row_scale, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_qmxfp4(const uint8_t *Wq, const uint8_t *We8m0, const float *x, float *y,
                              const float *residual, int N, int K, int B, void *stream)
{
    return gemv_entry(K2_MXFP4, Wq, We8m0, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_qq4s(const uint8_t *Wq, const float *Ws, const float *x, float *y,
                            const float *residual, int N, int K, int B, void *stream)
{
    return gemv_entry(K2_Q4S, Wq, Ws, x, y, residual, N, K, B, stream);
}

extern "C" int k2_gemv_f32(const float *W, const float *x, float *y, const float *residual,
                           int N, int K, int B, void *stream)
{
    return gemv_entry(K2_F32, W, nullptr, x, y, residual, N, K, B, stream);
}

// Fused projection forms of the decode step, x = GroupedRMSNorm(h).
static int norm_gemv_check(int wdt, const void *W, const void *S, const float *h, const float *gamma,
                           int groups, const float *y, int N, int K)
{
    if (!k2_ptr_ok(W) || !k2_ptr_ok(h) || !k2_ptr_ok(gamma) || !k2_ptr_ok(y)) return K2_EINVAL;
    if ((wdt == K2_FP8E4M3 || wdt == K2_MXFP4 || wdt == K2_Q4S) && !S) return K2_EINVAL;
    if (N <= 0 || K <= 0 || groups <= 0) return K2_EINVAL;
    if (wdt != K2_F32 && wdt != K2_BF16 && wdt != K2_FP8E4M3 && wdt != K2_MXFP4 && wdt != K2_Q4S)
        return K2_EUNSUPPORTED;
    if (K % 32 || K > K2_MAX_LDS_FLOATS || groups > K2_MAX_GROUPS || K % (4 * groups))
        return K2_EUNSUPPORTED;
    if (wdt == K2_Q4S && K % 64) return K2_EUNSUPPORTED;
    return K2_OK;
}

static GemvArgs norm_args(const void *W, const void *S, const float *h, const float *gamma, int groups,
                          float eps, float *y, int N, int K)
{
    GemvArgs a{};
    a.W = W;
    a.Sf = (const float *)S;
    a.S8 = (const uint8_t *)S;
    a.x = h;
    a.gamma = gamma;
    a.groups = groups;
    a.eps = eps;
    a.y = y;
    a.N = N;
    a.K = K;
    a.B = 1;
    return a;
}

extern "C" int k2_norm_gemv(k2_dtype wdt, const void *W, const void *S, const float *h,
                            const float *gamma, int groups, float eps, float *y, int N, int K,
                            void *stream)
{
    int rc = norm_gemv_check(wdt, W, S, h, gamma, groups, y, N, K);
    if (rc) return rc;
    return gemv_dispatch(wdt, norm_args(W, S, h, gamma, groups, eps, y, N, K), PRO_NORM, EPI_PLAIN,
                         k2_stream(stream));
}

extern "C" int k2_norm_gemv_swiglu(k2_dtype wdt, const void *W, const void *S, const float *h,
                                   const float *gamma, int groups, float eps, float *act, int inter,
                                   int K, void *stream)
{
    int rc = norm_gemv_check(wdt, W, S, h, gamma, groups, act, 2 * inter, K);
    if (rc) return rc;
    GemvArgs a = norm_args(W, S, h, gamma, groups, eps, act, 2 * inter, K);
    a.n_out = inter;
    return gemv_dispatch(wdt, a, PRO_NORM, EPI_SWIGLU, k2_stream(stream));
}

extern "C" int k2_norm_gemv_argmax(k2_dtype wdt, const void *W, const void *S, const float *h,
                                   const float *gamma, int groups, float eps, float *logits, int N,
                                   int K, int32_t *out_idx, void *ws, size_t ws_bytes, void *stream)
{
    int rc = norm_gemv_check(wdt, W, S, h, gamma, groups, logits, N, K);
    if (rc) return rc;
    if (!out_idx || !ws || ((uintptr_t)ws & 255u) || ws_bytes < argmax_ws_bytes()) return K2_EINVAL;
    GemvArgs a = norm_args(W, S, h, gamma, groups, eps, logits, N, K);
    argmax_ws_carve(ws, a.am);
    a.am.out_idx = out_idx;
    return gemv_dispatch(wdt, a, PRO_NORM, EPI_ARGMAX, k2_stream(stream));
}
