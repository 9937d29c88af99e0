// decode.hip -- one decode position of a dense decoder-only model, composed
// from the gfx950 kernels ([k2-burn] "Project layout": model.rs embed ->
// layers -> norm -> lm_head; layer.rs norm + attention residual, norm + MLP
// residual; mlp.rs SwiGLU).
//
// Per layer, five phases, each reading its weights exactly once:
//   1. GroupedRMSNorm (in the GEMV prologue) + QKV GEMV          -> qkv
//   2. RoPE + KV append at pos + split-K GQA attention + combine  -> o
//   3. O GEMV + residual                                          -> h
//   4. GroupedRMSNorm (prologue) + gate/up GEMV + SwiGLU          -> act
//   5. down GEMV + residual                                       -> h
// Phases 2 and 3 are one launch where the shape allows it (attn_then_o),
// so a layer is four or five kernels.  Then GroupedRMSNorm + lm_head GEMV +
// first-maximum argmax.  The embedding gather opens the step.  All
// activations are fp32.
//
// The position comes from the host (k2_decode_step) or from device memory
// (k2_decode_step_dev, whose last kernel advances it): the device form
// launches the same kernels with grids that do not depend on the position,
// so one captured step replays at every position.
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

struct DecodeWs {
    float *h, *qkv, *o, *act;
    void *attn;
    void *am;
    int32_t *next_scratch;
};

static size_t ws_layout(const k2_config *c, DecodeWs *w, void *base)
{
    const size_t qkv_rows = (size_t)(c->n_qh + 2 * c->n_kv) * c->head_dim;
    size_t off = 0;
    char *b = (char *)base;
    auto take = [&](size_t bytes) {
        char *p = b ? b + off : nullptr;
        off += k2_align256(bytes);
        return p;
    };
    char *h = take((size_t)c->hidden * 4);
    char *qkv = take(qkv_rows * 4);
    char *o = take((size_t)c->n_qh * c->head_dim * 4);
    char *act = take((size_t)c->inter * 4);
    char *attn = take(attn_ws_bytes(c->n_qh, c->n_kv, c->head_dim, c->cap));
    char *am = take(argmax_ws_bytes());
    char *nx = take(4);
    if (w) {
        w->h = (float *)h;
        w->qkv = (float *)qkv;
        w->o = (float *)o;
        w->act = (float *)act;
        w->attn = attn;
        w->am = am;
        w->next_scratch = (int32_t *)nx;
    }
    return off;
}

static bool mat_ok(int wdt, const void *w, const void *s)
{
    if (!k2_ptr_ok(w)) return false;
    if ((wdt == K2_FP8E4M3 || wdt == K2_MXFP4 || wdt == K2_Q4S) && !s) return false;
    return true;
}

static int config_check(const k2_config *c)
{
    if (!c) return K2_EINVAL;
    if (c->hidden <= 0 || c->n_layers <= 0 || c->n_qh <= 0 || c->n_kv <= 0 || c->head_dim <= 0 ||
        c->inter <= 0 || c->vocab <= 0 || c->groups <= 0 || c->cap <= 0 || !(c->eps >= 0.f) ||
        !(c->rope_theta > 0))
        return K2_EINVAL;
    if (c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
        return K2_EUNSUPPORTED;
    if (c->n_qh % c->n_kv) return K2_EUNSUPPORTED;
    const int rep = c->n_qh / c->n_kv;
    if (rep != 1 && rep != 2 && rep != 4 && rep != 8) return K2_EUNSUPPORTED;
    if (c->groups > K2_MAX_GROUPS || c->hidden % (4 * c->groups)) return K2_EUNSUPPORTED;
    const int qd = c->n_qh * c->head_dim;
    if (c->hidden % 32 || qd % 32 || c->inter % 32) return K2_EUNSUPPORTED;
    if (c->hidden > K2_MAX_LDS_FLOATS || qd > K2_MAX_LDS_FLOATS || c->inter > K2_MAX_LDS_FLOATS)
        return K2_EUNSUPPORTED;
    if (c->wdt != K2_F32 && c->wdt != K2_BF16 && c->wdt != K2_FP8E4M3 && c->wdt != K2_MXFP4 &&
        c->wdt != K2_Q4S)
        return K2_EUNSUPPORTED;
    if (c->wdt == K2_Q4S && (c->hidden % 64 || qd % 64 || c->inter % 64)) return K2_EUNSUPPORTED;
    if (c->kvdt != K2_F32 && c->kvdt != K2_BF16 && c->kvdt != K2_I8) return K2_EUNSUPPORTED;
    if (c->embdt != K2_F32 && c->embdt != K2_BF16) return K2_EUNSUPPORTED;
    if (c->cap > K2_ATTN_MAX_SPLITS * K2_ATTN_MAX_CHUNK) return K2_EUNSUPPORTED;
    return K2_OK;
}

static int model_check(const k2_model *m)
{
    if (!m) return K2_EINVAL;
    int rc = config_check(&m->cfg);
    if (rc) return rc;
    const k2_config *c = &m->cfg;
    if (!k2_ptr_ok(m->embed) || !k2_ptr_ok(m->g_final) || !k2_ptr_ok(m->rope) || !m->layers)
        return K2_EINVAL;
    if (!mat_ok(c->wdt, m->lm, m->lm_s)) return K2_EINVAL;
    if (!m->ws || ((uintptr_t)m->ws & 255u) || m->ws_bytes < ws_layout(c, nullptr, nullptr))
        return K2_EINVAL;
    for (int l = 0; l < c->n_layers; ++l) {
        const k2_layer *L = &m->layers[l];
        if (!mat_ok(c->wdt, L->qkv, L->qkv_s) || !mat_ok(c->wdt, L->o, L->o_s) ||
            !mat_ok(c->wdt, L->gu, L->gu_s) || !mat_ok(c->wdt, L->down, L->down_s))
            return K2_EINVAL;
        if (!k2_ptr_ok(L->g_in) || !k2_ptr_ok(L->g_post) || !k2_ptr_ok(L->kc) || !k2_ptr_ok(L->vc))
            return K2_EINVAL;
        if (c->kvdt == K2_I8 && (!k2_ptr_ok(L->ks) || !k2_ptr_ok(L->vs))) return K2_EINVAL;
    }
    return K2_OK;
}

// token / d_token: host token, or device token (d_token non-null).
// pos / d_pos: host position, or device position (d_pos non-null; advanced
// by one at the end of the step when it lies in [0, cap)).
static int decode_impl(const k2_model *m, int token, const int32_t *d_token, int pos, int32_t *d_pos,
                       float *logits, int32_t *next, int32_t *d_err, hipStream_t st)
{
    int rc = model_check(m);
    if (rc) return rc;
    const k2_config *c = &m->cfg;
    if (logits && !k2_aligned16(logits)) return K2_EINVAL;
    if (!d_pos && (pos < 0 || pos >= c->cap)) return K2_ERANGE;
    if (!d_token && (token < 0 || token >= c->vocab)) return K2_ERANGE;

    DecodeWs w;
    ws_layout(c, &w, m->ws);
    AttnArgs at{};
    attn_ws_carve(w.attn, c->n_qh, c->n_kv, c->head_dim, c->cap, at);
    ArgmaxArgs am{};
    argmax_ws_carve(w.am, am);

    const int H = c->hidden, hd = c->head_dim, wdt = c->wdt;
    const int qkv_rows = (c->n_qh + 2 * c->n_kv) * hd;

    rc = embed_launch(c->embdt, m->embed, H, c->vocab, d_token ? -1 : token, d_token, d_err, w.h, st);
    if (rc) return rc;

    at.qkv = w.qkv;
    at.cos_sin = m->rope;
    at.out = w.o;
    at.n_qh = c->n_qh;
    at.n_kv = c->n_kv;
    at.cap = c->cap;
    at.scale = 1.0f / sqrtf((float)hd);
    at.d_err = d_err;
    if (d_pos) {
        // the grid covers the most splits the capacity allows; the kernels
        // derive the position, length, chunk and split count from *d_pos
        at.d_pos = d_pos;
        at.S = attn_max_splits(c->n_kv, c->cap);
        at.chunk = 0;
        at.pos = 0;
        at.len = 1;
    } else {
        at.pos = pos;
        at.len = pos + 1;
        at.S = attn_splits(c->n_kv, at.len, &at.chunk);
    }

    for (int l = 0; l < c->n_layers; ++l) {
        const k2_layer *L = &m->layers[l];
        GemvArgs g{};
        g.W = L->qkv;
        g.Sf = (const float *)L->qkv_s;
        g.S8 = (const uint8_t *)L->qkv_s;
        g.x = w.h;
        g.gamma = L->g_in;
        g.eps = c->eps;
        g.groups = c->groups;
        g.y = w.qkv;
        g.N = qkv_rows;
        g.K = H;
        g.B = 1;
        if ((rc = gemv_dispatch(wdt, g, PRO_NORM, EPI_PLAIN, st))) return rc;

        at.kc = L->kc;
        at.vc = L->vc;
        at.ks = L->ks;
        at.vs = L->vs;

        GemvArgs o{};
        o.W = L->o;
        o.Sf = (const float *)L->o_s;
        o.S8 = (const uint8_t *)L->o_s;
        o.x = w.o;
        o.y = w.h;
        o.residual = w.h;
        o.N = H;
        o.K = c->n_qh * hd;
        o.B = 1;
        if ((rc = attn_then_o(wdt, c->kvdt, hd, c->n_qh / c->n_kv, at, o, d_err, st))) return rc;

        GemvArgs gu{};
        gu.W = L->gu;
        gu.Sf = (const float *)L->gu_s;
        gu.S8 = (const uint8_t *)L->gu_s;
        gu.x = w.h;
        gu.gamma = L->g_post;
        gu.eps = c->eps;
        gu.groups = c->groups;
        gu.y = w.act;
        gu.N = 2 * c->inter;
        gu.n_out = c->inter;
        gu.K = H;
        gu.B = 1;
        if ((rc = gemv_dispatch(wdt, gu, PRO_NORM, EPI_SWIGLU, st))) return rc;

        GemvArgs dn{};
        dn.W = L->down;
        dn.Sf = (const float *)L->down_s;
        dn.S8 = (const uint8_t *)L->down_s;
        dn.x = w.act;
        dn.y = w.h;
        dn.residual = w.h;
        dn.N = H;
        dn.K = c->inter;
        dn.B = 1;
        if ((rc = gemv_dispatch(wdt, dn, PRO_NONE, EPI_PLAIN, st))) return rc;
    }

    if (logits) {
        GemvArgs lm{};
        lm.W = m->lm;
        lm.Sf = (const float *)m->lm_s;
        lm.S8 = (const uint8_t *)m->lm_s;
        lm.x = w.h;
        lm.gamma = m->g_final;
        lm.eps = c->eps;
        lm.groups = c->groups;
        lm.y = logits;
        lm.N = c->vocab;
        lm.K = H;
        lm.B = 1;
        lm.am = am;
        lm.am.out_idx = next ? next : w.next_scratch;
        lm.am.adv_pos = d_pos;                      // the step's last kernel advances it
        lm.am.adv_cap = c->cap;
        return gemv_dispatch(wdt, lm, PRO_NORM, EPI_ARGMAX, st);
    }
    if (d_pos) return pos_advance_launch(d_pos, c->cap, st);
    return K2_OK;
}

}  // namespace k2

using namespace k2;

extern "C" size_t k2_decode_workspace_bytes(const k2_config *cfg)
{
    if (config_check(cfg)) return 0;
    return ws_layout(cfg, nullptr, nullptr);
}

extern "C" int k2_model_check(const k2_model *m) { return model_check(m); }

extern "C" int k2_decode_step(const k2_model *m, int token, int pos, float *logits,
                              int32_t *next_token, void *stream)
{
    return decode_impl(m, token, nullptr, pos, nullptr, logits, next_token, nullptr, k2_stream(stream));
}

extern "C" int k2_decode_step_dev(const k2_model *m, const int32_t *d_token, int32_t *d_pos,
                                  float *logits, int32_t *next_token, int32_t *d_err, void *stream)
{
    if (!d_token || !d_pos) return K2_EINVAL;
    return decode_impl(m, -1, d_token, -1, d_pos, logits, next_token, d_err, k2_stream(stream));
}
