// attn_rows.hip -- the attention of a prefill chunk in one launch: RoPE and
// cache append of the chunk's rows, then one query slice per position over
// the cache up to that position (the device code is in attn_impl.h).
// Kept in its own translation unit, apart from the decode attention
// launchers.
#include "attn_impl.h"

namespace k2 {

template <int KVDT, int REP>
static int attn_rows_go(const AttnArgs &a, int n_rows, int S_max, hipStream_t st)
{
    constexpr size_t lds = sizeof(float) * attn_stream_lds_floats<KVDT, 128, REP>();
    const int64_t part_stride = (int64_t)a.n_kv * S_max * REP * 128;
    const int64_t ml_stride = (int64_t)a.n_kv * S_max * REP * 2;
    hipLaunchKernelGGL((attn_rows_kernel<KVDT, 128, REP>), dim3(S_max, a.n_kv, n_rows), dim3(ATT_NT), lds, st,
                       a, n_rows, part_stride, ml_stride);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

template <int KVDT>
static int attn_rows_rep(int rep, const AttnArgs &a, int T, int S_max, hipStream_t st)
{
    switch (rep) {
    case 1: return attn_rows_go<KVDT, 1>(a, T, S_max, st);
    case 2: return attn_rows_go<KVDT, 2>(a, T, S_max, st);
    case 4: return attn_rows_go<KVDT, 4>(a, T, S_max, st);
    case 8: return attn_rows_go<KVDT, 8>(a, T, S_max, st);
    }
    return K2_EUNSUPPORTED;
}

size_t attn_rows_ws_bytes(int n_qh, int n_kv, int hd, int cap, int T)
{
    const size_t S = (size_t)attn_max_splits(n_kv, cap), rep = (size_t)(n_qh / n_kv);
    return k2_align256((size_t)T * n_kv * S * rep * hd * 4) + k2_align256((size_t)T * n_kv * S * rep * 2 * 4);
}

size_t attn_rows_cnt_bytes(int n_kv, int T) { return k2_align256((size_t)T * n_kv * 4); }

bool attn_rows_ok(int kvdt, int n_qh, int n_kv, int hd, int cap, int pos0, int T)
{
    if (hd != 128 || T < 1 || n_kv < 1 || n_qh % n_kv) return false;
    const int rep = n_qh / n_kv;
    if (rep != 1 && rep != 2 && rep != 4 && rep != 8) return false;
    if (kvdt != K2_F32 && kvdt != K2_BF16 && kvdt != K2_I8) return false;
    int chunk = 0;
    return (size_t)attn_splits(n_kv * T, pos0 + T, &chunk) <= (size_t)attn_max_splits(n_kv, cap);
}

int attn_rows_launch(int kvdt, const float *qkv, const float *cos_sin, float *qrot, float *out, void *kc,
                     void *vc, float *ks, float *vs, int n_qh, int n_kv, int hd, int cap, int pos0, int T,
                     void *ws, unsigned *cnt, hipStream_t st, uint16_t *oh, uint16_t *ol, bool *planes,
                     bool appended)
{
    if (planes) *planes = false;
    if (!attn_rows_ok(kvdt, n_qh, n_kv, hd, cap, pos0, T)) return K2_EUNSUPPORTED;
    const int rep = n_qh / n_kv;
    switch (appended ? -1 : kvdt) {
    case -1: break;                            // q rotated and the rows appended by the QKV product
    case K2_F32:
        hipLaunchKernelGGL((rope_append_rows_kernel<K2_F32, 128>), dim3(n_kv, T), dim3(K2_BLOCK), 0, st, qkv,
                           cos_sin, qrot, kc, vc, ks, vs, n_qh, n_kv, cap, pos0);
        break;
    case K2_BF16:
        hipLaunchKernelGGL((rope_append_rows_kernel<K2_BF16, 128>), dim3(n_kv, T), dim3(K2_BLOCK), 0, st, qkv,
                           cos_sin, qrot, kc, vc, ks, vs, n_qh, n_kv, cap, pos0);
        break;
    case K2_I8:
        hipLaunchKernelGGL((rope_append_rows_kernel<K2_I8, 128>), dim3(n_kv, T), dim3(K2_BLOCK), 0, st, qkv,
                           cos_sin, qrot, kc, vc, ks, vs, n_qh, n_kv, cap, pos0);
        break;
    default: return K2_EUNSUPPORTED;
    }
    K2_CHECK_LAUNCH();
    // chunks of a bf16 / int8 cache with enough rows: every row's attention
    // on the matrix cores, the K/V tiles shared by the rows of a block
    const bool mc = T >= ATTN_PREFILL_MIN_T ||
                    (T >= ATTN_PREFILL_LONG_MIN_T && (int64_t)pos0 + T > ATTN_PREFILL_LONG_LEN);
    const size_t S = (size_t)attn_max_splits(n_kv, cap);
    char *p = (char *)ws;
    float *part = (float *)p;
    p += k2_align256((size_t)T * n_kv * S * rep * hd * 4);
    float *part_ml = (float *)p;
    if (mc && (kvdt == K2_BF16 || kvdt == K2_I8)) {
        const int rc = attn_prefill_launch(kvdt, qrot, out, kc, vc, ks, vs, n_qh, n_kv, hd, cap, pos0, T, part,
                                           part_ml, (int)S, cnt, oh, ol, st);
        if (rc == K2_OK && planes && oh && ol) *planes = true;
        return rc;
    }
    AttnArgs a{};
    a.part = part;
    a.part_ml = part_ml;
    a.head_cnt = cnt;
    a.q = qrot;
    a.kc = kc;
    a.vc = vc;
    a.ks = ks;
    a.vs = vs;
    a.out = out;
    a.n_qh = n_qh;
    a.n_kv = n_kv;
    a.cap = cap;
    a.len = pos0 + T;                          // the last slice's length
    a.pos = a.len - 1;
    a.scale = 1.0f / sqrtf((float)hd);
    // the decode rule's block target shared by the T rows: every row gets
    // 1/T of the splits one decode position would (8 rows at 528 positions:
    // 4 splits of 132 instead of 9 of 64, one round of 256 blocks)
    const int S_max = attn_splits(n_kv * T, a.len, &a.chunk);
    switch (kvdt) {
    case K2_F32: return attn_rows_rep<K2_F32>(rep, a, T, S_max, st);
    case K2_BF16: return attn_rows_rep<K2_BF16>(rep, a, T, S_max, st);
    default: return attn_rows_rep<K2_I8>(rep, a, T, S_max, st);
    }
}

}  // namespace k2
