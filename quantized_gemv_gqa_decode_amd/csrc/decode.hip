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
// The environment variable K2_PERSISTENT=1 runs the position as one
// cooperative launch of the persistent step kernel instead (step_impl.h),
// for the shapes it is instantiated for.  It is not the default: on MI355X a
// grid barrier (about 3 us with its data hand-off) costs more than the gap
// between two dependent kernels (about 2.5 us), and the persistent form
// measures slower on the 3.7B-shaped workload.
#include <stdlib.h>
#include <string.h>

#include "k2_dev.h"
#include "k2_internal.h"
#include "step_impl.h"
#include "fused_impl.h"

namespace k2 {

int step_dispatch_f32(int, int, int, const StepArgs &, int, int, int, int, hipStream_t);
int step_dispatch_bf16(int, int, int, const StepArgs &, int, int, int, int, hipStream_t);
int step_dispatch_fp8(int, int, int, const StepArgs &, int, int, int, int, hipStream_t);
int step_dispatch_mxfp4(int, int, int, const StepArgs &, int, int, int, int, hipStream_t);

// fused.hip
struct FusedArgs;
bool fused_ok(int hd, int rep, int n_kv, int hidden, int n_qh_hd);
int fused_qao_launch(int wdt, int kvdt, const FusedArgs &f, hipStream_t st);
int fused_zero_sync(unsigned *sync, int words, hipStream_t st);

struct DecodeWs {
    float *h, *qkv, *o, *act;
    unsigned *fsync;            // per-layer counters of the fused QKV+attention+O kernel
    void *attn;
    void *am;
    int32_t *next_scratch;
    k2_layer *layers_dev;       // device copy of the layer table (persistent kernel)
    unsigned *sync;             // its barrier and arrival counters
    float *trail;               // its write-once activation trail
};

// per-layer slice of the persistent kernel's activation trail:
// [qkv | attention output | residual after O | SwiGLU | residual after down],
// each part 256-byte aligned
struct TrailLayout {
    int off_qkv, off_o, off_ha, off_act, off_hb;
    int64_t layer_floats;
};

static TrailLayout trail_layout(const k2_config *c)
{
    auto al = [](int64_t n) { return (n + 63) & ~(int64_t)63; };
    TrailLayout t{};
    int64_t o = 0;
    t.off_qkv = (int)o; o += al((int64_t)(c->n_qh + 2 * c->n_kv) * c->head_dim);
    t.off_o = (int)o;   o += al((int64_t)c->n_qh * c->head_dim);
    t.off_ha = (int)o;  o += al(c->hidden);
    t.off_act = (int)o; o += al(c->inter);
    t.off_hb = (int)o;  o += al(c->hidden);
    t.layer_floats = o;
    return t;
}

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
    char *lt = take((size_t)c->n_layers * sizeof(k2_layer));
    char *sy = take((size_t)STEP_SYNC_WORDS * sizeof(unsigned));
    const TrailLayout tl = trail_layout(c);
    char *tr = take(((size_t)((c->hidden + 63) & ~63) + (size_t)c->n_layers * tl.layer_floats) * 4);
    char *fs = take((size_t)c->n_layers * FUSE_SYNC_WORDS * sizeof(unsigned));
    if (w) {
        w->fsync = (unsigned *)fs;
        w->trail = (float *)tr;
        w->layers_dev = (k2_layer *)lt;
        w->sync = (unsigned *)sy;
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

// The layer table travels in the kernel arguments (no host staging, no
// host synchronisation); the launch carrying the first chunk also clears
// the persistent kernel's counters.
constexpr int TABLE_CHUNK = 24;
struct TableChunk {
    k2_layer L[TABLE_CHUNK];
    k2_layer *dst;
    unsigned *sync;
    int first, count;
};

__global__ void step_prologue_kernel(const TableChunk c)
{
    const int t = threadIdx.x;
    constexpr int W = sizeof(k2_layer) / sizeof(uint64_t);
    static_assert(sizeof(k2_layer) % sizeof(uint64_t) == 0, "k2_layer layout");
    const uint64_t *src = reinterpret_cast<const uint64_t *>(c.L);
    uint64_t *dst = reinterpret_cast<uint64_t *>(c.dst + c.first);
    for (int i = t; i < c.count * W; i += blockDim.x) dst[i] = src[i];
    if (c.sync)
        for (int i = t; i < STEP_SYNC_WORDS; i += blockDim.x) c.sync[i] = 0u;
}

// The fused QKV + attention + O kernel is opt-in (K2_FUSED=1): measured on
// the 3.7B shape it saves ~1 % with bf16 KV and loses ~6 % with int8 KV (its
// attention role sets the register budget of every block of the launch).
static bool fused_enabled()
{
    const char *e = getenv("K2_FUSED");
    return e && strcmp(e, "1") == 0;
}

static bool persistent_enabled()
{
    const char *e = getenv("K2_PERSISTENT");
    return e && strcmp(e, "1") == 0;
}

static int device_coop_ok()
{
    int dev = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) return 0;
    return coop;
}

// K2_EUNSUPPORTED: no persistent kernel for this shape (nothing enqueued).
static int decode_persistent(const k2_model *m, const DecodeWs &w, const AttnArgs &at0,
                             const ArgmaxArgs &am, int token, const int32_t *d_token, int pos,
                             float *logits, int32_t *next, int32_t *d_err, hipStream_t st)
{
    const k2_config *c = &m->cfg;
    const int rep = c->n_qh / c->n_kv;
    if (c->n_kv > STEP_MAX_KV) return K2_EUNSUPPORTED;
    if (!((c->head_dim == 128 || c->head_dim == 16) && (rep == 2 || rep == 4))) return K2_EUNSUPPORTED;
    if (!device_coop_ok()) return K2_EUNSUPPORTED;

    StepArgs A{};
    A.layers = w.layers_dev;
    A.embed = m->embed;
    A.lm = m->lm;
    A.lm_s = m->lm_s;
    A.g_final = m->g_final;
    A.rope = m->rope;
    const TrailLayout tl = trail_layout(c);
    A.trail = w.trail;
    A.layer_floats = tl.layer_floats;
    A.off_qkv = tl.off_qkv;
    A.off_o = tl.off_o;
    A.off_ha = tl.off_ha;
    A.off_act = tl.off_act;
    A.off_hb = tl.off_hb;
    A.logits = logits;
    A.part = at0.part;
    A.part_ml = at0.part_ml;
    A.am_v = am.part_v;
    A.am_i = am.part_i;
    A.next = next ? next : w.next_scratch;
    A.d_token = d_token;
    A.d_err = d_err;
    A.sync = w.sync;
    A.token = token;
    A.pos = pos;
    A.len = pos + 1;
    A.n_layers = c->n_layers;
    A.H = c->hidden;
    A.inter = c->inter;
    A.vocab = c->vocab;
    A.groups = c->groups;
    A.n_qh = c->n_qh;
    A.n_kv = c->n_kv;
    A.cap = c->cap;
    A.embdt = c->embdt;
    A.attn_S = attn_splits_fine(c->n_kv, c->cap, A.len, &A.attn_chunk);
    A.eps = c->eps;
    A.scale = 1.0f / sqrtf((float)c->head_dim);

    const int qd = c->n_qh * c->head_dim;
    // probe: is there an instantiation?  (a dispatch with an impossible
    // block budget would still launch, so check the shape table first)
    switch (c->wdt) {
    case K2_F32: case K2_BF16: case K2_FP8E4M3: case K2_MXFP4: break;
    default: return K2_EUNSUPPORTED;
    }
    for (int first = 0; first < c->n_layers; first += TABLE_CHUNK) {
        TableChunk tc{};
        tc.first = first;
        tc.count = c->n_layers - first < TABLE_CHUNK ? c->n_layers - first : TABLE_CHUNK;
        memcpy(tc.L, m->layers + first, (size_t)tc.count * sizeof(k2_layer));
        tc.dst = w.layers_dev;
        tc.sync = first == 0 ? w.sync : nullptr;
        hipLaunchKernelGGL(step_prologue_kernel, dim3(1), dim3(256), 0, st, tc);
        K2_CHECK_LAUNCH();
    }
    const int max_blocks = K2_ARGMAX_MAX_BLOCKS;
    switch (c->wdt) {
    case K2_F32: return step_dispatch_f32(c->kvdt, c->head_dim, rep, A, c->hidden, qd, c->inter, max_blocks, st);
    case K2_BF16: return step_dispatch_bf16(c->kvdt, c->head_dim, rep, A, c->hidden, qd, c->inter, max_blocks, st);
    case K2_FP8E4M3: return step_dispatch_fp8(c->kvdt, c->head_dim, rep, A, c->hidden, qd, c->inter, max_blocks, st);
    default: return step_dispatch_mxfp4(c->kvdt, c->head_dim, rep, A, c->hidden, qd, c->inter, max_blocks, st);
    }
}

static int decode_impl(const k2_model *m, int token, const int32_t *d_token, int pos, float *logits,
                       int32_t *next, int32_t *d_err, hipStream_t st)
{
    int rc = model_check(m);
    if (rc) return rc;
    const k2_config *c = &m->cfg;
    if (logits && !k2_aligned16(logits)) return K2_EINVAL;
    if (pos < 0 || pos >= c->cap) return K2_ERANGE;
    if (!d_token && (token < 0 || token >= c->vocab)) return K2_ERANGE;

    DecodeWs w;
    ws_layout(c, &w, m->ws);
    AttnArgs at{};
    attn_ws_carve(w.attn, c->n_qh, c->n_kv, c->head_dim, c->cap, at);
    ArgmaxArgs am{};
    argmax_ws_carve(w.am, am);

    if (persistent_enabled()) {
        rc = decode_persistent(m, w, at, am, d_token ? -1 : token, d_token, pos, logits, next,
                               d_err, st);
        if (rc != K2_EUNSUPPORTED) return rc;
    }

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
    at.pos = pos;
    at.len = pos + 1;
    at.scale = 1.0f / sqrtf((float)hd);
    at.S = attn_splits(c->n_kv, at.len, &at.chunk);
    const bool fused = fused_enabled() && wdt != K2_Q4S &&
                       fused_ok(hd, c->n_qh / c->n_kv, c->n_kv, H, c->n_qh * hd);
    if (fused && (rc = fused_zero_sync(w.fsync, c->n_layers * FUSE_SYNC_WORDS, st))) return rc;

    for (int l = 0; l < c->n_layers; ++l) {
        const k2_layer *L = &m->layers[l];
        if (fused) {
            FusedArgs f{};
            f.q.W = L->qkv;
            f.q.Sf = (const float *)L->qkv_s;
            f.q.S8 = (const uint8_t *)L->qkv_s;
            f.q.x = w.h;
            f.q.gamma = L->g_in;
            f.q.eps = c->eps;
            f.q.groups = c->groups;
            f.q.y = w.qkv;
            f.q.N = qkv_rows;
            f.q.K = H;
            f.q.B = 1;
            f.o.W = L->o;
            f.o.Sf = (const float *)L->o_s;
            f.o.S8 = (const uint8_t *)L->o_s;
            f.o.x = w.o;
            f.o.y = w.h;
            f.o.residual = w.h;
            f.o.N = H;
            f.o.K = c->n_qh * hd;
            f.o.B = 1;
            f.at = at;
            f.at.kc = L->kc;
            f.at.vc = L->vc;
            f.at.ks = L->ks;
            f.at.vs = L->vs;
            f.sync = w.fsync + (size_t)l * FUSE_SYNC_WORDS;
            f.d_err = d_err;
            if ((rc = fused_qao_launch(wdt, c->kvdt, f, st))) return rc;
        } else {
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
        }

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
        if ((rc = gemv_dispatch(wdt, lm, PRO_NORM, EPI_ARGMAX, st))) return rc;
    }
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
    return decode_impl(m, token, nullptr, pos, logits, next_token, nullptr, k2_stream(stream));
}

extern "C" int k2_decode_step_dev(const k2_model *m, const int32_t *d_token, int pos, float *logits,
                                  int32_t *next_token, int32_t *d_err, void *stream)
{
    if (!d_token) return K2_EINVAL;
    return decode_impl(m, -1, d_token, pos, logits, next_token, d_err, k2_stream(stream));
}
