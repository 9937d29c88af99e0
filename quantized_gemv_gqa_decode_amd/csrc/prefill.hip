// prefill.hip -- a chunk of prompt positions through the whole model in one
// sweep, the projections on the matrix cores.
//
// [k2-burn] "Working end to end" names prefill beside single-token decode:
// the prompt is consumed before the first decode step, and consuming it
// position by position gives exactly the incremental (cached) result.  With
// T positions at once every projection is a [N][K] x [K][T] product, so a
// weight byte feeds 2T flops: past a few positions that is a dense
// contraction, run here on v_mfma_f32_16x16x32_bf16 by the product of
// gemm_mfma.hip (activations split into bf16 hi + lo, fp32 accumulation;
// fp8, MXFP4 and Q4S weights decoded in registers to exact bf16 values with
// their scales applied to the sums), which reads the weights once for up to
// 256 positions.
//
// Per layer, for the T rows of the chunk:
//   1. GroupedRMSNorm of every row                       (one launch)
//   2. QKV = W_qkv X                                     (matrix cores)
//   3. RoPE and KV append of every row, then every row's attention over
//      [0, pos0 + t] (one launch for head_dim 128; else per position, in
//      order, so that position t sees the K/V rows of the earlier ones)
//   4. H += W_o O                                        (matrix cores, add)
//   5. GroupedRMSNorm, then ACT = silu(W_g X) * (W_u X)  (matrix cores, SwiGLU)
//   6. H += W_d ACT                                      (matrix cores, add)
// then the final norm, lm_head and first-maximum argmax of the LAST row only
// (the GEMV of the decode step).
#include <stdlib.h>
#include <string.h>

#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

constexpr int PF_MAX_T = GM_MAX_T;         // positions per call
constexpr int VF_MAX_T = 32;               // positions per verification call (its lm_head keeps [T][vocab])

struct PfTokens {
    int tok[PF_MAX_T];
};

// h[t] = E[tok[t]] (bf16 widened exactly, or fp32), t < T
__global__ void embed_rows_kernel(const PfTokens tk, int embdt, const void *E, int H, float *h)
{
    const int t = blockIdx.y;
    const int64_t base = (int64_t)tk.tok[t] * H;
    float *dst = h + (int64_t)t * H;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < H; i += gridDim.x * blockDim.x)
        dst[i] = embdt == K2_BF16 ? bf16_to_f32(((const uint16_t *)E)[base + i]) : ((const float *)E)[base + i];
}

struct PrefillWs {
    float *h, *x, *qkv, *o, *act, *part, *qrot, *lm_part, *logits, *ar_v;
    float *sq;                     // [T][hidden / 64] sums of squares of the residual stream
    uint16_t *xh, *xl, *ah, *al;   // bf16 hi / lo planes: norm / attention outputs, SwiGLU output
    int *ar_i;
    void *attn, *rows, *am;
    unsigned *rows_cnt, *dm_cnt;
    int32_t *next;
};

// First maximum of every row of x [rows][n] in two launches: block (b, t)
// of the first finds the first maximum of the b-th of AR_NB contiguous
// slices of row t; one wave per row then takes the first maximum of the
// AR_NB candidates (ties go to the lower index at both levels, so the result
// is the row's first maximum).
constexpr int AR_NB = K2_WAVE;

__global__ __launch_bounds__(K2_BLOCK) void argmax_rows_part_kernel(const float *x, int n, float *pv, int *pi)
{
    const int t = blockIdx.y, b = blockIdx.x;
    const int per = (n + AR_NB - 1) / AR_NB;
    const int lo = b * per, hi = lo + per < n ? lo + per : n;
    const float *r = x + (int64_t)t * n;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    // 16 elements per thread loaded before the first comparison (one memory
    // round trip per 4096 of the slice; the winner does not depend on order)
    constexpr int AB = 16;
    for (int i0 = lo; i0 < hi; i0 += AB * K2_BLOCK) {
        float v[AB];
#pragma unroll
        for (int u = 0; u < AB; ++u) {
            const int i = i0 + u * K2_BLOCK + (int)threadIdx.x;
            v[u] = i < hi ? r[i] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < AB; ++u) {
            const int i = i0 + u * K2_BLOCK + (int)threadIdx.x;
            if (i < hi) argmax_pair_max(bv, bi, v[u], i);
        }
    }
    argmax_block(bv, bi);
    if (threadIdx.x == 0) {
        pv[t * AR_NB + b] = bv;
        pi[t * AR_NB + b] = bi;
    }
}

__global__ __launch_bounds__(K2_WAVE) void argmax_rows_final_kernel(const float *pv, const int *pi, int32_t *out)
{
    const int t = blockIdx.x, lane = threadIdx.x;
    float v = pv[t * AR_NB + lane];
    int i = pi[t * AR_NB + lane];
    argmax_wave(v, i);
    if (lane == 0) out[t] = i;
}

// A projection of the chunk's T rows: for bf16 weights up to 32 rows the
// small-T product (dense_mfma.hip, measured faster there), else the
// token-blocked GEMM (gemm_mfma.hip), which reads every weight byte from
// HBM once per call and decodes quantized weights in registers.
constexpr int PF_GEMM_MIN_T = 33;

static bool pf_dense(int wdt, int T) { return wdt == K2_BF16 && T < PF_GEMM_MIN_T; }

static size_t pf_proj_bytes(int wdt, int N, int K, int T, int epi)
{
    return pf_dense(wdt, T) ? dense_mfma_ws_bytes(N, K, T) : gemm_mfma_ws_bytes(wdt, N, K, T, epi);
}

static int pf_proj(int wdt, const void *W, const void *Ws, const float *x, float *y, int N, int K, int T, int epi,
                   float *ws, unsigned *cnt, hipStream_t st, const DmNorm &nrm = DmNorm{}, float *osq = nullptr)
{
    if (pf_dense(wdt, T)) return dense_mfma((const uint16_t *)W, x, y, N, K, T, epi, ws, st, cnt, nrm, osq);
    if (nrm.gamma || osq) return K2_EINVAL;     // the norm travels in the small-T product only
    return gemm_mfma(wdt, W, Ws, x, y, N, K, T, epi, ws, st);
}

// the projections' scratch for any chunk of up to T rows (the split count
// of a product, and so its partials, need not grow with T)
static size_t pf_part_bytes(const k2_config *c, int T)
{
    const int qkv_rows = (c->n_qh + 2 * c->n_kv) * c->head_dim, qd = c->n_qh * c->head_dim;
    const int wd = c->wdt;
    size_t m = 0;
    for (int t = 2; t <= T; ++t) {
        const size_t b[4] = {pf_proj_bytes(wd, qkv_rows, c->hidden, t, DM_EPI_PLAIN),
                             pf_proj_bytes(wd, c->hidden, qd, t, DM_EPI_ADD),
                             pf_proj_bytes(wd, 2 * c->inter, c->hidden, t, DM_EPI_SWIGLU),
                             pf_proj_bytes(wd, c->hidden, c->inter, t, DM_EPI_ADD)};
        for (size_t v : b) m = v > m ? v : m;
    }
    return m;
}

// verify: also the lm_head of every row (matrix-core partials and, for a
// caller that passes no logits buffer, the [T][vocab] logits)
static size_t pf_layout(const k2_config *c, int T, PrefillWs *w, void *base, bool verify = false)
{
    const size_t qkv_rows = (size_t)(c->n_qh + 2 * c->n_kv) * c->head_dim, qd = (size_t)c->n_qh * c->head_dim;
    size_t off = 0;
    char *b = (char *)base;
    auto take = [&](size_t bytes) {
        char *p = b ? b + off : nullptr;
        off += k2_align256(bytes);
        return p;
    };
    // the parts that must stay zero between calls (the attention's split
    // counters, the argmax's) come first, at offsets that do not depend on T:
    // a workspace sized for one T serves every smaller T
    char *attn = take(attn_ws_bytes(c->n_qh, c->n_kv, c->head_dim, c->cap));
    char *rows_cnt = take(attn_rows_cnt_bytes(c->n_kv, PF_MAX_T));
    char *am = take(argmax_ws_bytes());
    char *nx = take(4);
    // arrival counters of the small-T products' in-kernel reduction (one per
    // 64-row block of the tallest product)
    {
        int rows = c->vocab;
        const int prod[3] = {(c->n_qh + 2 * c->n_kv) * c->head_dim, 2 * c->inter, c->hidden};
        for (int r : prod) rows = r > rows ? r : rows;
        char *dc = take((size_t)dense_mfma_cnt_words(rows) * 4);
        if (w) w->dm_cnt = (unsigned *)dc;
    }
    char *rows = take(attn_rows_ws_bytes(c->n_qh, c->n_kv, c->head_dim, c->cap, T));
    char *h = take((size_t)T * c->hidden * 4);
    char *x = take((size_t)T * c->hidden * 4);
    char *qkv = take((size_t)T * qkv_rows * 4);
    char *o = take((size_t)T * qd * 4);
    char *act = take((size_t)T * c->inter * 4);
    char *part = take(pf_part_bytes(c, T));
    char *qrot = take((size_t)T * qd * 4);
    char *sq = take((size_t)T * (c->hidden / 64 + 1) * 4);
    // activation planes for the token-blocked products: every row a token
    // block may read (T rounded up to 128)
    const size_t prow = (size_t)(T + 127) / 128 * 128;
    const size_t xw = (size_t)c->hidden > qd ? (size_t)c->hidden : qd;
    char *xh = take(prow * xw * 2);
    char *xl = take(prow * xw * 2);
    char *ah = take(prow * (size_t)c->inter * 2);
    char *al = take(prow * (size_t)c->inter * 2);
    char *lm_part = verify ? take(c->wdt == K2_BF16 ? dense_mfma_ws_bytes(c->vocab, c->hidden, T)
                                                    : gemm_mfma_ws_bytes(c->wdt, c->vocab, c->hidden, T, DM_EPI_PLAIN))
                           : nullptr;
    char *lgt = verify ? take((size_t)T * c->vocab * 4) : nullptr;
    char *arv = verify ? take((size_t)T * AR_NB * 4) : nullptr;
    char *ari = verify ? take((size_t)T * AR_NB * 4) : nullptr;
    if (w) {
        w->ar_v = (float *)arv;
        w->ar_i = (int *)ari;
        w->lm_part = (float *)lm_part;
        w->logits = (float *)lgt;
        w->rows = rows;
        w->rows_cnt = (unsigned *)rows_cnt;
        w->qrot = (float *)qrot;
        w->sq = (float *)sq;
        w->xh = (uint16_t *)xh;
        w->xl = (uint16_t *)xl;
        w->ah = (uint16_t *)ah;
        w->al = (uint16_t *)al;
        w->h = (float *)h;
        w->x = (float *)x;
        w->qkv = (float *)qkv;
        w->o = (float *)o;
        w->act = (float *)act;
        w->part = (float *)part;
        w->attn = attn;
        w->am = am;
        w->next = (int32_t *)nx;
    }
    return off;
}

// Shapes this path handles (K2_EUNSUPPORTED otherwise): bf16, fp8, MXFP4 or
// Q4S projection weights whose products the matrix-core kernels take.
static int pf_shape_ok(const k2_config *c, bool verify = false)
{
    const int wd = c->wdt;
    if (wd != K2_BF16 && wd != K2_FP8E4M3 && wd != K2_MXFP4 && wd != K2_Q4S) return K2_EUNSUPPORTED;
    if (verify && !(wd == K2_BF16 ? dense_mfma_ok(c->vocab, c->hidden)
                                  : gemm_mfma_ok(c->vocab, c->hidden, DM_EPI_PLAIN)))
        return K2_EUNSUPPORTED;
    const int qkv_rows = (c->n_qh + 2 * c->n_kv) * c->head_dim, qd = c->n_qh * c->head_dim;
    if (wd == K2_BF16 && (!dense_mfma_ok(qkv_rows, c->hidden) || !dense_mfma_ok(c->hidden, qd) ||
                          !dense_mfma_ok(2 * c->inter, c->hidden) || !dense_mfma_ok(c->hidden, c->inter)))
        return K2_EUNSUPPORTED;
    if (!gemm_mfma_ok(qkv_rows, c->hidden, DM_EPI_PLAIN) || !gemm_mfma_ok(c->hidden, qd, DM_EPI_ADD) ||
        !gemm_mfma_ok(2 * c->inter, c->hidden, DM_EPI_SWIGLU) || !gemm_mfma_ok(c->hidden, c->inter, DM_EPI_ADD))
        return K2_EUNSUPPORTED;
    return K2_OK;
}

// The matrix-core products read MXFP4 scale bytes four at a time and Q4S
// block scales two at a time: their scale arrays must be 16-byte aligned.
static bool pf_scales_ok(const k2_model *m)
{
    const k2_config *c = &m->cfg;
    if (c->wdt != K2_MXFP4 && c->wdt != K2_Q4S) return true;
    if (!k2_ptr_ok(m->lm_s)) return false;
    for (int l = 0; l < c->n_layers; ++l) {
        const k2_layer *L = &m->layers[l];
        if (!k2_ptr_ok(L->qkv_s) || !k2_ptr_ok(L->o_s) || !k2_ptr_ok(L->gu_s) || !k2_ptr_ok(L->down_s))
            return false;
    }
    return true;
}

// verify: logits [T][vocab] (nullable: kept in the workspace) and next [T]
// (required) for every row; else logits [vocab] and next of the last row.
static int prefill_impl(const k2_model *m, const int32_t *tokens, int T, int pos0, float *logits,
                        int32_t *next, void *ws, size_t ws_bytes, bool verify, hipStream_t st)
{
    int rc = k2_model_check(m);
    if (rc) return rc;
    const k2_config *c = &m->cfg;
    if (T < 2 || T > (verify ? VF_MAX_T : PF_MAX_T)) return K2_EUNSUPPORTED;
    if (!tokens || (verify && !k2_ptr_ok(next))) return K2_EINVAL;
    if ((rc = pf_shape_ok(c, verify))) return rc;
    if (!pf_scales_ok(m)) return K2_EINVAL;
    if (logits && !k2_aligned16(logits)) return K2_EINVAL;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < pf_layout(c, T, nullptr, nullptr, verify)) return K2_EINVAL;
    if (pos0 < 0 || (int64_t)pos0 + T > c->cap) return K2_ERANGE;
    PfTokens tk{};
    for (int t = 0; t < T; ++t) {
        if (tokens[t] < 0 || tokens[t] >= c->vocab) return K2_ERANGE;
        tk.tok[t] = tokens[t];
    }

    PrefillWs w;
    pf_layout(c, T, &w, ws, verify);
    const int H = c->hidden, hd = c->head_dim, I = c->inter, rep = c->n_qh / c->n_kv;
    const int qkv_rows = (c->n_qh + 2 * c->n_kv) * hd, qd = c->n_qh * hd;

    int blocks = (H + K2_BLOCK - 1) / K2_BLOCK;
    if (blocks > 16) blocks = 16;
    hipLaunchKernelGGL(embed_rows_kernel, dim3(blocks, T), dim3(K2_BLOCK), 0, st, tk, c->embdt, m->embed,
                       H, w.h);
    K2_CHECK_LAUNCH();

    // the chunk's attention as one launch (hd 128), else per position
    AttnArgs at{};
    attn_ws_carve(w.attn, c->n_qh, c->n_kv, hd, c->cap, at);
    at.cos_sin = m->rope;
    at.n_qh = c->n_qh;
    at.n_kv = c->n_kv;
    at.cap = c->cap;
    at.scale = 1.0f / sqrtf((float)hd);

    // Token-blocked products (above 32 bf16 rows, and every quantized
    // format) read their activations as bf16 hi / lo planes: the row norms,
    // the matrix-core attention and the SwiGLU epilogue write them directly,
    // so no split launch runs before those products.
    const bool planes = !pf_dense(c->wdt, T);
    // Small-T products (bf16, up to 32 rows) take the row norms in their
    // activation staging: every product that adds into the residual stream
    // (O, down) also writes its 64-row sums of squares, from which the next
    // product (gate/up, the next layer's QKV, the lm_head) scales h.  Only
    // the first layer's input norm, after the embedding, runs on its own.
    const bool fnorm = !planes && dense_norm_ok(H, c->groups);
    auto norm_of = [&](const float *gamma) {
        DmNorm n;
        n.gamma = gamma;
        n.nsq = w.sq;
        n.groups = c->groups;
        n.eps = c->eps;
        return n;
    };
    float *osq = fnorm ? w.sq : nullptr;
    for (int l = 0; l < c->n_layers; ++l) {
        const k2_layer *L = &m->layers[l];
        bool appended = false;                   // the QKV product rotated q and appended the rows
        if (planes) {
            if ((rc = rmsnorm_rows_planes_launch(w.h, L->g_in, w.xh, w.xl, T, H, c->groups, c->eps, st))) return rc;
            if ((rc = gemm_mfma_planes(c->wdt, L->qkv, L->qkv_s, w.xh, w.xl, w.qkv, nullptr, nullptr, qkv_rows, H,
                                       T, DM_EPI_PLAIN, w.part, st)))
                return rc;
        } else {
            // small-T bf16: the product's last blocks also rotate q and k and
            // append the chunk's rows to the cache where they sum the partials
            // (head_dim 128), else the attention launch does
            DmNorm nrm;
            const float *xin = w.x;
            if (fnorm && l > 0) {
                nrm = norm_of(L->g_in);
                xin = w.h;
            } else if ((rc = rmsnorm_rows_launch(w.h, L->g_in, w.x, T, H, c->groups, c->eps, st))) {
                return rc;
            }
            DmRope rp;
            rp.cs = m->rope;
            rp.qrot = w.qrot;
            rp.kc = L->kc;
            rp.vc = L->vc;
            rp.ks = L->ks;
            rp.vs = L->vs;
            rp.n_qh = c->n_qh;
            rp.n_kv = c->n_kv;
            rp.cap = c->cap;
            rp.pos0 = pos0;
            rp.kvdt = c->kvdt;
            rc = attn_rows_ok(c->kvdt, c->n_qh, c->n_kv, hd, c->cap, pos0, T)
                     ? dense_mfma((const uint16_t *)L->qkv, xin, w.qkv, qkv_rows, H, T, DM_EPI_PLAIN, w.part, st,
                                  w.dm_cnt, nrm, nullptr, &rp)
                     : K2_EUNSUPPORTED;
            appended = rc == K2_OK;
            if (rc == K2_EUNSUPPORTED)
                rc = pf_proj(c->wdt, L->qkv, L->qkv_s, xin, w.qkv, qkv_rows, H, T, DM_EPI_PLAIN, w.part, w.dm_cnt,
                             st, nrm);
            if (rc) return rc;
        }
        at.kc = L->kc;
        at.vc = L->vc;
        at.ks = L->ks;
        at.vs = L->vs;
        bool o_planes = false;                       // the attention wrote its output as planes (w.xh / w.xl)
        rc = attn_rows_launch(c->kvdt, w.qkv, m->rope, w.qrot, w.o, L->kc, L->vc, L->ks, L->vs, c->n_qh,
                              c->n_kv, hd, c->cap, pos0, T, w.rows, w.rows_cnt, st, planes ? w.xh : nullptr,
                              planes ? w.xl : nullptr, &o_planes, appended);
        if (rc && rc != K2_EUNSUPPORTED) return rc;
        const bool per_position = rc == K2_EUNSUPPORTED;
        for (int t = 0; per_position && t < T; ++t) {
            at.qkv = w.qkv + (int64_t)t * qkv_rows;
            at.out = w.o + (int64_t)t * qd;
            at.pos = pos0 + t;
            at.len = at.pos + 1;
            at.S = attn_splits(c->n_kv, at.len, &at.chunk);
            if ((rc = attn_launch(c->kvdt, hd, rep, true, at, st))) return rc;
        }
        if (o_planes)
            rc = gemm_mfma_planes(c->wdt, L->o, L->o_s, w.xh, w.xl, w.h, nullptr, nullptr, H, qd, T, DM_EPI_ADD,
                                  w.part, st);
        else
            rc = pf_proj(c->wdt, L->o, L->o_s, w.o, w.h, H, qd, T, DM_EPI_ADD, w.part, w.dm_cnt, st, DmNorm{}, osq);
        if (rc) return rc;
        if (planes) {
            if ((rc = rmsnorm_rows_planes_launch(w.h, L->g_post, w.xh, w.xl, T, H, c->groups, c->eps, st)))
                return rc;
            if ((rc = gemm_mfma_planes(c->wdt, L->gu, L->gu_s, w.xh, w.xl, nullptr, w.ah, w.al, 2 * I, H, T,
                                       DM_EPI_SWIGLU, w.part, st)))
                return rc;
            if ((rc = gemm_mfma_planes(c->wdt, L->down, L->down_s, w.ah, w.al, w.h, nullptr, nullptr, H, I, T,
                                       DM_EPI_ADD, w.part, st)))
                return rc;
        } else if (fnorm) {
            if ((rc = pf_proj(c->wdt, L->gu, L->gu_s, w.h, w.act, 2 * I, H, T, DM_EPI_SWIGLU, w.part, w.dm_cnt,
                              st, norm_of(L->g_post))))
                return rc;
            if ((rc = pf_proj(c->wdt, L->down, L->down_s, w.act, w.h, H, I, T, DM_EPI_ADD, w.part, w.dm_cnt, st,
                              DmNorm{}, osq)))
                return rc;
        } else {
            if ((rc = rmsnorm_rows_launch(w.h, L->g_post, w.x, T, H, c->groups, c->eps, st))) return rc;
            if ((rc = pf_proj(c->wdt, L->gu, L->gu_s, w.x, w.act, 2 * I, H, T, DM_EPI_SWIGLU, w.part, w.dm_cnt,
                              st)))
                return rc;
            if ((rc = pf_proj(c->wdt, L->down, L->down_s, w.act, w.h, H, I, T, DM_EPI_ADD, w.part, w.dm_cnt, st)))
                return rc;
        }
    }

    if (verify) {
        // every row: final norm, lm_head on the matrix cores, first-maximum argmax
        float *lg = logits ? logits : w.logits;
        if (fnorm) {
            rc = dense_mfma((const uint16_t *)m->lm, w.h, lg, c->vocab, H, T, DM_EPI_PLAIN, w.lm_part, st, w.dm_cnt,
                            norm_of(m->g_final));
        } else {
            if ((rc = rmsnorm_rows_launch(w.h, m->g_final, w.x, T, H, c->groups, c->eps, st))) return rc;
            rc = c->wdt == K2_BF16 ? dense_mfma((const uint16_t *)m->lm, w.x, lg, c->vocab, H, T, DM_EPI_PLAIN,
                                                w.lm_part, st, w.dm_cnt)
                                   : gemm_mfma(c->wdt, m->lm, m->lm_s, w.x, lg, c->vocab, H, T, DM_EPI_PLAIN,
                                               w.lm_part, st);
        }
        if (rc) return rc;
        hipLaunchKernelGGL(argmax_rows_part_kernel, dim3(AR_NB, T), dim3(K2_BLOCK), 0, st, lg, c->vocab, w.ar_v,
                           w.ar_i);
        K2_CHECK_LAUNCH();
        hipLaunchKernelGGL(argmax_rows_final_kernel, dim3(T), dim3(K2_WAVE), 0, st, w.ar_v, w.ar_i, next);
        K2_CHECK_LAUNCH();
    } else if (logits) {
        ArgmaxArgs am{};
        argmax_ws_carve(w.am, am);
        GemvArgs lm{};
        lm.W = m->lm;
        lm.Sf = (const float *)m->lm_s;            // fp8 row scales, Q4S block scales
        lm.S8 = (const uint8_t *)m->lm_s;          // MXFP4 E8M0 bytes
        lm.x = w.h + (int64_t)(T - 1) * H;
        lm.gamma = m->g_final;
        lm.eps = c->eps;
        lm.groups = c->groups;
        lm.y = logits;
        lm.N = c->vocab;
        lm.K = H;
        lm.B = 1;
        lm.am = am;
        lm.am.out_idx = next ? next : w.next;
        if ((rc = gemv_dispatch(c->wdt, lm, PRO_NORM, EPI_ARGMAX, st))) return rc;
    }
    return K2_OK;
}

}  // namespace k2

using namespace k2;

extern "C" size_t k2_prefill_workspace_bytes(const k2_config *cfg, int T)
{
    if (!cfg || T < 2 || T > PF_MAX_T || pf_shape_ok(cfg)) return 0;
    if (k2_decode_workspace_bytes(cfg) == 0) return 0;
    return pf_layout(cfg, T, nullptr, nullptr);
}

extern "C" int k2_prefill(const k2_model *m, const int32_t *tokens, int T, int pos0, float *logits,
                          int32_t *next_token, void *ws, size_t ws_bytes, void *stream)
{
    return prefill_impl(m, tokens, T, pos0, logits, next_token, ws, ws_bytes, false, k2_stream(stream));
}

extern "C" size_t k2_verify_workspace_bytes(const k2_config *cfg, int T)
{
    if (!cfg || T < 2 || T > VF_MAX_T || pf_shape_ok(cfg, true)) return 0;
    if (k2_decode_workspace_bytes(cfg) == 0) return 0;
    return pf_layout(cfg, T, nullptr, nullptr, true);
}

extern "C" int k2_verify(const k2_model *m, const int32_t *tokens, int T, int pos0, float *logits,
                         int32_t *next_tokens, void *ws, size_t ws_bytes, void *stream)
{
    return prefill_impl(m, tokens, T, pos0, logits, next_tokens, ws, ws_bytes, true, k2_stream(stream));
}
