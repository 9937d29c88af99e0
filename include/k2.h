/*
 * k2.h -- C ABI of libk2.so: the batch-1 decode hot path of a dense
 * decoder-only LLM (and the routed-expert GEMV of a latent-MoE layer) on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [k2-burn]      README of k2-burn, the K2-Horizon port: "Model shape",
 *                  "Working end to end" (GroupedRMSNorm, split-half RoPE, GQA,
 *                  SwiGLU MLP; "prefill + single-token decode" over "a
 *                  preallocated per-layer KV cache"), "KV cache storage"
 *                  (int8 with a per-head_dim-block scale; a prompt that does
 *                  not fit is rejected), "Quantization" (fp8 E4M3 Linear
 *                  weights), "Limitations" (effective batch size 1; plain
 *                  SDPA with the softmax in fp32).
 *   [k3_run.c]     kimi-k3-in-c src/cli/k3_run.c: header comment (token ids
 *                  in, token ids out; routed experts multiplied straight out
 *                  of MXFP4), real_cfg_hardcoded() (latent MoE: 896 experts,
 *                  top-16, 2 shared, latent 3584, inter 3072, routed_scale,
 *                  renorm, latent_norm), forward() (on failure the logits are
 *                  left untouched and the caller must check), the request
 *                  validation in main() (refuse rather than clamp), argmax_()
 *                  (first maximum wins).
 *   [cpu_weights.rs] avarok_core kimi_k3 cpu_weights.rs: MoeWeights (down, up,
 *                  norm, router, bias, experts (w1, w2, w3), shared).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless a comment says "host".  Every call
 *   only enqueues work on `stream` (a hipStream_t passed as void*; NULL is the
 *   null stream) and returns without synchronizing.
 * - The caller owns and allocates every buffer (weights, caches, activations,
 *   workspaces).  The library allocates no device memory, keeps no pointer
 *   after returning, and holds no mutable global state.  Calls on different
 *   streams with disjoint buffers may run concurrently.
 * - Activations are fp32.  bf16 values travel as uint16_t bit patterns; fp8
 *   is OCP E4M3FN (uint8_t codes); MXFP4 is OCP E2M1 elements packed two per
 *   byte, low nibble = even column, with one E8M0 scale byte per 32
 *   consecutive columns of a row.
 * - Matrices are row-major [N out][K in].
 * - Errors: every int-returning call returns a k2_status.  Arguments are
 *   validated on the host (scalars and pointer alignment only, no device
 *   sync).  On K2_EINVAL / K2_ERANGE / K2_EUNSUPPORTED nothing is enqueued and
 *   every output buffer is left untouched.  K2_EHIP (a launch error reported
 *   by the HIP runtime) is the only status after which outputs are undefined.
 * - Alignment: weight, cache and activation pointers must be 16-byte
 *   aligned (the kernels use 128-bit loads); K2_EINVAL otherwise.
 */
#ifndef K2_H
#define K2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define K2_ABI_VERSION 2

typedef enum {
    K2_OK = 0,
    K2_EINVAL = -1,        /* null / misaligned pointer, non-positive size */
    K2_ERANGE = -2,        /* token, position or length out of range */
    K2_EUNSUPPORTED = -3,  /* a shape or dtype this build does not handle */
    K2_EHIP = -4           /* the HIP runtime reported a launch error */
} k2_status;

typedef enum {
    K2_F32 = 0,
    K2_BF16 = 1,
    K2_FP8E4M3 = 2,
    K2_MXFP4 = 3,
    K2_I8 = 4,
    K2_Q4S = 5             /* int4 weights, one fp32 scale per 64 columns */
} k2_dtype;

int k2_abi_version(void);
/* Host string for a status code (static storage). */
const char *k2_status_str(int status);

/* ------------------------------------------------------------------------
 * Weight preparation ([k2-burn] "Quantization": only Linear weights are
 * quantized; [k3_run.c] header: experts in MXFP4).  Input is the bf16 draw.
 * ---------------------------------------------------------------------- */

/* fp8 E4M3FN with one fp32 scale per output row:
 *   row_scale[n] = fp32(max_k |W[n][k]| / 448),
 *   codes[n][k]  = E4M3FN round-to-nearest-even, saturating at +-448, of
 *                  fp32(W[n][k] / row_scale[n]); an all-zero row has scale 0
 *                  and codes 0.  The sign of a zero result is kept.
 * W: uint16 bf16 [N][K]; codes: uint8 [N][K]; row_scale: float [N].
 * K2_EINVAL if K % 16 or any pointer is null/misaligned. */
int k2_quantize_fp8_rows(const uint16_t *W, uint8_t *codes, float *row_scale,
                         int N, int K, void *stream);

/* MXFP4 (OCP Microscaling: E2M1 elements, blocks of 32, E8M0 scale):
 *   e_b  = clamp(unbiased exponent field of fp32 amax_b - 2, -127, 127),
 *   e8m0[n][b] = e_b + 127,
 *   code = E2M1 round-to-nearest-even, saturating at +-6, of W * 2^-e_b.
 * W: uint16 bf16 [N][K]; q: uint8 [N][K/2]; e8m0: uint8 [N][K/32].
 * K2_EUNSUPPORTED if K % 32 != 0. */
/* Q4S ([k2-burn] "Working end to end" / "Quantization": int4 "Q4S" with
 * block size 64; the pages give no more, the reading taken is symmetric
 * int4 with one fp32 scale per block):
 *   a = max |W| over 64 consecutive columns of a row, s[n][b] = fp32(a / 7),
 *   code = clamp(rint(fp32(W / s)), -7, 7) (ties to even; two's complement
 *   nibble, -8 never written), a = 0 gives s = 0 and codes 0.
 * W: uint16 bf16 [N][K]; q: uint8 [N][K/2] (low nibble = even column);
 * s: float [N][K/64].  K2_EUNSUPPORTED if K % 64 != 0. */
int k2_quantize_q4s(const uint16_t *W, uint8_t *q, float *s, int N, int K, void *stream);

int k2_quantize_mxfp4(const uint16_t *W, uint8_t *q, uint8_t *e8m0, int N, int K,
                      void *stream);

/* ------------------------------------------------------------------------
 * Step operations
 * ---------------------------------------------------------------------- */

/* GroupedRMSNorm ([k2-burn] "Model shape": layernorm_num_groups).  For each
 * of `rows` vectors of length `hidden`, cut into `groups` equal contiguous
 * groups: y = x / sqrt(mean over the group of x^2 + eps) * gamma (gamma over
 * the full hidden size).  x, y: [rows][hidden] (may alias); gamma: [hidden].
 * K2_EUNSUPPORTED if hidden % groups != 0 or hidden / groups > 16384. */
int k2_rmsnorm_grouped(const float *x, const float *gamma, float *y, int rows, int hidden,
                       int groups, float eps, void *stream);

/* Dequantizing GEMV, y[b][n] = sum_k W_hat[n][k] * x[b][k] (+ residual[b][n]),
 * fp32 accumulation, for B activation vectors (1 <= B <= 8).
 *   qbf16:  W uint16 bf16 [N][K]
 *   qfp8:   W uint8 E4M3FN [N][K], row_scale float [N] (applied after the sum)
 *   qmxfp4: Wq uint8 [N][K/2], We8m0 uint8 [N][K/32] (per-block scale
 *           applied to each 32-column partial sum)
 *   qq4s:   Wq uint8 [N][K/2], Ws float [N][K/64] (per-block scale applied
 *           to each block's partial sum; K % 64 == 0)
 *   f32:    W float [N][K]
 * x: [B][K]; y: [B][N]; residual (nullable): [B][N], may alias y.
 * K2_EUNSUPPORTED if K % 32 != 0 (K % 64 for Q4S) or B * K > 12288. */
int k2_gemv_qq4s(const uint8_t *Wq, const float *Ws, const float *x, float *y,
                 const float *residual, int N, int K, int B, void *stream);
int k2_gemv_qbf16(const uint16_t *W, const float *x, float *y, const float *residual,
                  int N, int K, int B, void *stream);
int k2_gemv_qfp8(const uint8_t *W, const float *row_scale, const float *x, float *y,
                 const float *residual, int N, int K, int B, void *stream);
int k2_gemv_qmxfp4(const uint8_t *Wq, const uint8_t *We8m0, const float *x, float *y,
                   const float *residual, int N, int K, int B, void *stream);
int k2_gemv_f32(const float *W, const float *x, float *y, const float *residual, int N,
                int K, int B, void *stream);

/* Fused projection forms used by k2_decode_step (one kernel each), with
 * x = GroupedRMSNorm(h; gamma, groups, eps) computed in the prologue:
 *   k2_norm_gemv:        y = W_hat x                       (QKV projection)
 *   k2_norm_gemv_swiglu: act = silu(W_hat[0:inter] x) * W_hat[inter:2 inter] x
 *                        ([k2-burn] SwiGLU MLP: gate rows, then up rows)
 *   k2_norm_gemv_argmax: logits = W_hat x and out_idx = first-maximum argmax
 *                        (final norm + untied lm_head); ws as k2_argmax.
 * W/S in the formats of the k2_gemv_* calls (S: row scales for fp8, E8M0 for
 * MXFP4, NULL otherwise).  h: [K]; K % 32 == 0, K <= 12288, groups <= 8,
 * K % (4 groups) == 0. */
int k2_norm_gemv(k2_dtype wdt, const void *W, const void *S, const float *h, const float *gamma,
                 int groups, float eps, float *y, int N, int K, void *stream);
int k2_norm_gemv_swiglu(k2_dtype wdt, const void *W, const void *S, const float *h,
                        const float *gamma, int groups, float eps, float *act, int inter, int K,
                        void *stream);
int k2_norm_gemv_argmax(k2_dtype wdt, const void *W, const void *S, const float *h,
                        const float *gamma, int groups, float eps, float *logits, int N, int K,
                        int32_t *out_idx, void *ws, size_t ws_bytes, void *stream);

/* RoPE table for split-half rotary embedding ([k2-burn] "Working end to
 * end"; the table is sized by the context window, "KV cache storage"):
 * cos_sin[p][i][0] = cos(p * theta^(-2i/head_dim)), [1] = sin(...), for
 * p < cap, i < head_dim/2, computed in fp64 on the device and stored fp32. */
int k2_rope_table(float *cos_sin, int cap, int head_dim, double theta, void *stream);

/* Split-half RoPE in place on n_qh query heads q [n_qh][hd] and n_kv key heads
 * k [n_kv][hd] at position pos: element i pairs with i + hd/2,
 *   u_i <- a cos - b sin,  u_{i+hd/2} <- a sin + b cos.
 * K2_ERANGE if pos >= cap; K2_EUNSUPPORTED unless hd is 16, 32, 64 or 128. */
int k2_rope(float *q, float *k, const float *cos_sin, int n_qh, int n_kv, int head_dim,
            int pos, int cap, void *stream);

/* Store one position of K and V ([k2-burn] "KV cache storage").  Caches are
 * [n_kv][cap][hd]; k, v are fp32 [n_kv][hd].
 *   k2_kv_append:      kvdt K2_F32 (stored as is) or K2_BF16 (round to
 *                      nearest even).
 *   k2_kv_append_int8: symmetric int8 per (kv head, position) block:
 *                      s = fp32(max|x| / 127), code = clamp(rint(fp32(x / s)),
 *                      -127, 127); max|x| = 0 gives s = 0 and codes 0.
 *                      Scales ks, vs: [n_kv][cap] fp32.
 * K2_ERANGE if pos >= cap. */
int k2_kv_append(k2_dtype kvdt, const float *k, const float *v, void *kc, void *vc,
                 int n_kv, int head_dim, int cap, int pos, void *stream);
int k2_kv_append_int8(const float *k, const float *v, int8_t *kc, int8_t *vc, float *ks,
                      float *vs, int n_kv, int head_dim, int cap, int pos, void *stream);

/* GQA decode attention ([k2-burn] "Model shape": 4x KV repeat; "Limitations":
 * plain SDPA with the softmax in fp32).  For query head h the key/value head
 * is h / (n_qh / n_kv); out[h] = softmax(q_h . K[0..len) * scale) V[0..len).
 * Split over positions with an online fp32 softmax and a fixed-order combine
 * (run-to-run deterministic).  kvdt: K2_F32, K2_BF16 or K2_I8 (ks, vs
 * required).  q: [n_qh][hd] (already rotated); out: [n_qh][hd].
 * ws: workspace of k2_attn_workspace_bytes(n_qh, n_kv, head_dim, cap) bytes,
 * zero-filled by the caller before its first use (the kernels leave it zeroed
 * again on exit); calls that share a workspace must not overlap in time.  K2_ERANGE unless 1 <= len <= cap; K2_EUNSUPPORTED unless
 * hd is 16/32/64/128 and n_qh / n_kv is 1, 2, 4 or 8. */
size_t k2_attn_workspace_bytes(int n_qh, int n_kv, int head_dim, int cap);
int k2_gqa_decode_attn(k2_dtype kvdt, const float *q, const void *kc, const void *vc,
                       const float *ks, const float *vs, float *out, int n_qh, int n_kv,
                       int head_dim, int cap, int len, float scale, void *ws, size_t ws_bytes,
                       void *stream);

/* k2_gqa_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and the same kernels, with the
 * workspace in a file-scope device array of the library
 * (k2_gqa_decode_attn_scratch_limit() bytes, 4 MiB; one copy per device,
 * held until the process ends) instead of a caller buffer.  The call
 * allocates nothing.  K2_EUNSUPPORTED when k2_attn_workspace_bytes(n_qh,
 * n_kv, head_dim, cap) exceeds the limit (nothing enqueued); otherwise the
 * refusals of k2_gqa_decode_attn, and K2_EHIP if the array's device address
 * cannot be obtained.  Every call on one device shares that device's array:
 * calls that overlap in time on one device (other streams, other host
 * threads) race and must be serialized by the caller. */
size_t k2_gqa_decode_attn_scratch_limit(void);
int k2_gqa_decode_attn_noalloc(k2_dtype kvdt, const float *q, const void *kc, const void *vc,
                               const float *ks, const float *vs, float *out, int n_qh, int n_kv,
                               int head_dim, int cap, int len, float scale, void *stream);

/* Fused step used by k2_decode_step: from the raw QKV projection
 * qkv = [q (n_qh*hd); k (n_kv*hd); v (n_kv*hd)], rotate q and k at `pos`,
 * store k and v at slot `pos` of the cache (kvdt as above), then attend over
 * slots [0, pos] with scale 1/sqrt(hd).  The stored values are the ones
 * attended to.  out: [n_qh][hd].  Same workspace as k2_gqa_decode_attn. */
int k2_rope_append_attn(k2_dtype kvdt, const float *qkv, const float *cos_sin, void *kc,
                        void *vc, float *ks, float *vs, float *out, int n_qh, int n_kv,
                        int head_dim, int cap, int pos, void *ws, size_t ws_bytes,
                        void *stream);

/* k2_rope_append_attn followed by the O projection with its residual
 * ([k2-burn] "Project layout": layer.rs, attention residual):
 *   h[n] += sum_k Wo[n][k] * out[k],  n < hidden, k < n_qh * head_dim.
 * wdt, Wo and Wo_s as for k2_gemv_q* / k2_gemv_f32 (Wo [hidden][n_qh*hd];
 * Wo_s: fp32 row scales for K2_FP8E4M3, E8M0 bytes for K2_MXFP4, fp32
 * block scales for K2_Q4S, NULL
 * otherwise).  out receives the attention output as in k2_rope_append_attn;
 * h is read and written in place.  Where the shape has one (fp32 or bf16
 * cache, head_dim 128, 4 query heads per kv head, n_qh*hd <= 4096, and the
 * attention and O grids fit the device at once) this is ONE launch whose O
 * blocks stream their weights while the attention runs; otherwise the
 * attention kernel and the GEMV.  Either way h is bit-identical to k2_rope_append_attn followed by
 * the GEMV.  d_err (device int32, nullable): set to K2_EHIP if a wait inside
 * the launch times out (outputs then undefined).  Same workspace as
 * k2_gqa_decode_attn; K2_EUNSUPPORTED unless n_qh*hd % 32 == 0 and
 * n_qh*hd <= 12288. */
int k2_rope_append_attn_o(k2_dtype kvdt, const float *qkv, const float *cos_sin, void *kc,
                          void *vc, float *ks, float *vs, float *out, int n_qh, int n_kv,
                          int head_dim, int cap, int pos, k2_dtype wdt, const void *Wo,
                          const void *Wo_s, float *h, int hidden, void *ws, size_t ws_bytes,
                          int32_t *d_err, void *stream);

/* Seeded sampling of one token from logits [vocab] ([k2-burn] "Project
 * layout": sampling.rs; "Usage": --top-k / --top-p / --min-p as separate
 * truncation filters, --repetition-penalty on already-seen tokens; the order
 * is the conventional one, the pages give none):
 * repetition penalty r on the distinct ids of prev (l > 0 -> l / r, else
 * l * r), temperature, top-k (ties: lower id first; top_k = 0: off, every
 * token stays a candidate), softmax, top-p (the shortest prefix whose
 * probability reaches top_p), min-p (keep p >= min_p * max p), then the first
 * kept token whose cumulative probability exceeds u * the kept total,
 * u = (word 0 of Philox4x32-10(counter = (counter lo, counter hi, 0, 0),
 * key = (seed lo, seed hi))) >> 8) * 2^-24.
 * logits: device float [vocab], vocab <= 2^24, read only; prev: device int32
 * [n_prev] (nullable when n_prev = 0; any length, repeats count once, ids
 * outside the vocabulary are ignored); out_token: device int32.
 * sp (host): 0 < temperature, top_k >= 0, 0 < top_p <= 1, 0 <= min_p < 1,
 * repetition_penalty >= 1 (K2_EINVAL otherwise).  1 <= top_k <= 64 with at
 * most 64 previous ids (and vocab <= 262144) takes a selection of the
 * k + n_prev best logits sorted by one wave; anything else the
 * whole-vocabulary path (radix selection by exact fixed-point probability
 * mass, no sort).  Greedy decoding is k2_argmax.  ws: device,
 * k2_sample_workspace_bytes(vocab) bytes, 256-byte aligned (no state kept
 * between calls). */
typedef struct {
    float temperature;
    int top_k;
    float top_p;
    float min_p;
    float repetition_penalty;
} k2_sampling;
size_t k2_sample_workspace_bytes(int vocab);
int k2_sample(const float *logits, int vocab, const k2_sampling *sp, const int32_t *prev, int n_prev,
              uint64_t seed, uint64_t counter, int32_t *out_token, void *ws, size_t ws_bytes,
              void *stream);

/* First-maximum argmax of x[0..n) ([k3_run.c] argmax_()): out_idx[0] is the
 * lowest index holding the largest value.  ws: k2_argmax_workspace_bytes(n)
 * bytes, zero-filled before first use (left zeroed on exit); calls that share
 * a workspace must not overlap in time. */
size_t k2_argmax_workspace_bytes(int n);
int k2_argmax(const float *x, int n, int32_t *out_idx, void *ws, size_t ws_bytes,
              void *stream);

/* ------------------------------------------------------------------------
 * Whole decode step of a dense decoder ([k2-burn] "Project layout": model.rs
 * embed -> layers -> norm -> lm_head; layer.rs norm + attention residual,
 * norm + MLP residual; mlp.rs SwiGLU)
 * ---------------------------------------------------------------------- */

typedef struct {
    int hidden, n_layers, n_qh, n_kv, head_dim, inter, vocab, groups, cap;
    float eps;
    double rope_theta;
    k2_dtype wdt;    /* projections + lm_head: K2_F32, K2_BF16, K2_FP8E4M3, K2_MXFP4, K2_Q4S */
    k2_dtype kvdt;   /* K2_F32, K2_BF16, K2_I8 */
    k2_dtype embdt;  /* K2_F32 or K2_BF16 */
} k2_config;

/* One layer (host struct of device pointers).  qkv stacks the q rows, then k,
 * then v; gu stacks the gate rows, then the up rows.  *_s: fp32 row scales
 * [N] (fp8), E8M0 bytes [N][K/32] (MXFP4), fp32 block scales [N][K/64]
 * (Q4S), NULL otherwise. */
typedef struct {
    const void *qkv, *qkv_s;    /* [(n_qh + 2 n_kv) hd][hidden] */
    const void *o, *o_s;        /* [hidden][n_qh hd] */
    const void *gu, *gu_s;      /* [2 inter][hidden] */
    const void *down, *down_s;  /* [hidden][inter] */
    const float *g_in, *g_post; /* [hidden] */
    void *kc, *vc;              /* [n_kv][cap][hd] of kvdt */
    float *ks, *vs;             /* [n_kv][cap] (int8 only) */
} k2_layer;

typedef struct {
    k2_config cfg;
    const void *embed;          /* [vocab][hidden] of embdt */
    const void *lm, *lm_s;      /* [vocab][hidden] of wdt (+ scales) */
    const float *g_final;       /* [hidden] */
    const float *rope;          /* k2_rope_table(cap, head_dim, rope_theta) */
    const k2_layer *layers;     /* HOST array [n_layers] */
    void *ws;                   /* k2_decode_workspace_bytes(&cfg), zero-filled
                                   before first use */
    size_t ws_bytes;
} k2_model;

size_t k2_decode_workspace_bytes(const k2_config *cfg);

/* Validate a model description (sizes, dtypes, pointers, alignment). */
int k2_model_check(const k2_model *m);

/* Prefill of T prompt positions pos0 .. pos0+T-1 in one sweep ([k2-burn]
 * "Working end to end": prefill + single-token decode).  Same result as T
 * calls of k2_decode_step at those positions, up to rounding: the
 * projections of the T rows run on the matrix cores with each fp32
 * activation split into bf16 hi + lo (about 16 significant bits, fp32
 * accumulation); fp8, MXFP4 and Q4S weights are decoded to exact bf16
 * values (fp8: the code's value, row scale applied to the row's sum; MXFP4:
 * the element times its block's 2^e; Q4S: the code, each 64-column block's
 * sum times its scale).  The caches receive every position; logits
 * (nullable) and next_token (nullable) are those of the LAST position.
 * tokens: HOST array [T].  Needs bf16, fp8, MXFP4 or Q4S projection weights
 * with hidden, n_qh * head_dim and inter multiples of 128, and 2 <= T <= 256
 * (K2_EUNSUPPORTED otherwise; a single position is k2_decode_step; MXFP4
 * and Q4S scale arrays 16-byte aligned, K2_EINVAL otherwise); every
 * weight byte is read from HBM once per call (the token blocks of a row
 * block, 32 to 128 positions each, share it through L2).  ws: device workspace of k2_prefill_workspace_bytes(&m->cfg, T) bytes
 * (it serves every smaller T), 256-byte aligned, zero-filled before its
 * first use (left zeroed where it must be); calls that share it must not
 * overlap in time.  K2_ERANGE if a token is outside the
 * vocabulary or pos0 + T > cap (nothing enqueued). */
size_t k2_prefill_workspace_bytes(const k2_config *cfg, int T);
int k2_prefill(const k2_model *m, const int32_t *tokens, int T, int pos0, float *logits,
               int32_t *next_token, void *ws, size_t ws_bytes, void *stream);

/* Batched greedy verification of T positions in one sweep (speculative
 * decoding: the pages' drafter proposes tokens and one pass over the
 * weights checks them all): the k2_prefill computation, plus the final norm,
 * the lm_head (matrix cores, any of k2_prefill's weight formats) and the
 * first-maximum argmax of EVERY row.
 * next_tokens[t] (device int32 [T], required) is the greedy token after
 * position pos0 + t, the same as a k2_decode_step at that position would
 * give up to rounding; logits (nullable, device [T][vocab]) receives every
 * row's logits.  A caller feeding [last accepted, d_1 .. d_{T-1}] accepts
 * d_i while d_i == next_tokens[i - 1]; cache slots past the accepted ones
 * are simply written again by later calls.  ws: k2_verify_workspace_bytes
 * (it includes the lm_head partials and a logits buffer), zero-filled
 * before its first use.  Same refusals as k2_prefill, with 2 <= T <= 32;
 * K2_EINVAL without next_tokens. */
size_t k2_verify_workspace_bytes(const k2_config *cfg, int T);
int k2_verify(const k2_model *m, const int32_t *tokens, int T, int pos0, float *logits,
              int32_t *next_tokens, void *ws, size_t ws_bytes, void *stream);

/* One decode position: embed `token` (host int), run every layer at `pos`
 * (its K and V are stored at slot pos before attending), then, when `logits`
 * is non-NULL, the final norm, the lm_head and the argmax.  logits: [vocab]
 * fp32 (nullable: prefill positions skip the head); next_token: device int32
 * (nullable), the first-maximum argmax.  K2_ERANGE if token is outside
 * [0, vocab) or pos outside [0, cap): refuse rather than clamp ([k3_run.c]
 * main()), nothing enqueued. */
int k2_decode_step(const k2_model *m, int token, int pos, float *logits, int32_t *next_token,
                   void *stream);

/* Same step with the token AND the position read from device memory, so
 * that a greedy loop runs without a host round trip and one captured step
 * (or a captured loop of steps) replays at every position:
 *   d_token (device int32, required): the token to embed; it may be the
 *     previous step's next_token.
 *   d_pos (device int32, required): the position; the step's last kernel
 *     advances it by one, so consecutive calls walk pos, pos + 1, ...
 * The launch grids do not depend on the position (the attention grid covers
 * the most splits the capacity allows; blocks past the position's split
 * count leave at once).  Range errors are caught on the device, where no
 * refusal before launch is possible ([k3_run.c] forward(): the caller must
 * check): a token outside [0, vocab) sets *d_err (device int32, nullable)
 * to K2_ERANGE and the step runs on token 0; a position outside [0, cap)
 * sets *d_err to K2_ERANGE, no cache slot is written, *d_pos is not
 * advanced, and logits / next_token are then undefined.  The caller must
 * read d_err before trusting the outputs.  K2_EINVAL (nothing enqueued) if
 * d_token or d_pos is NULL; otherwise the host-side refusals of
 * k2_decode_step. */
int k2_decode_step_dev(const k2_model *m, const int32_t *d_token, int32_t *d_pos, float *logits,
                       int32_t *next_token, int32_t *d_err, void *stream);

/* ------------------------------------------------------------------------
 * Latent-MoE layer ([k3_run.c] real_cfg_hardcoded(): n_experts 896, top-16,
 * 2 shared experts, latent 3584, moe inter 3072, routed_scale, renorm,
 * latent_norm; [cpu_weights.rs] MoeWeights: down, up, norm, router, bias,
 * experts (w1, w2, w3), shared).  T token rows are independent.
 * ---------------------------------------------------------------------- */

/* Router: logits = W_r x (bf16 [n_experts][hidden]), sigma = sigmoid(logits);
 * topk_idx[t] = the top_k experts by sigma + bias (bias: fp32 [n_experts],
 * nullable = zeros; it affects the selection only), in descending order with
 * the lower expert id first on equal scores; topk_w[t][j] = routed_scale *
 * sigma_j / (sum of the selected sigma).  x: [T][hidden]; outputs [T][top_k]
 * (int32 and fp32).  hidden % 32 == 0, hidden <= 12288, n_experts <= 1024,
 * top_k <= min(32, n_experts).  ws: k2_moe_route_workspace_bytes(T,
 * n_experts) bytes, 256-byte aligned. */
size_t k2_moe_route_workspace_bytes(int T, int n_experts);
int k2_moe_route(const uint16_t *Wr, const float *bias, const float *x, int T, int hidden,
                 int n_experts, int top_k, float routed_scale, int32_t *topk_idx, float *topk_w,
                 void *ws, size_t ws_bytes, void *stream);

/* Routed experts, gathered by expert ([k3_run.c]: routed experts multiplied
 * directly from MXFP4):
 *   r[t] = sum over j < top_k, in slot order, of
 *          topk_w[t][j] * W2_e (silu(W1_e z[t]) * (W3_e z[t])),  e = topk_idx[t][j].
 * z: [T][latent] fp32; r: [T][latent] fp32, overwritten.  Expert weights are
 * MXFP4 (format above) for all n_experts experts back to back:
 *   w13q [n_experts][2 inter][latent/2], w13s [n_experts][2 inter][latent/32]
 *        (rows 0..inter-1 are W1 (gate), rows inter..2 inter-1 are W3 (up)),
 *   w2q  [n_experts][latent][inter/2],   w2s  [n_experts][latent][inter/32].
 * Only the selected experts are read.  An expert id outside [0, n_experts)
 * is detected on the device: *d_err (device int32, nullable) is set to
 * K2_ERANGE and that slot contributes nothing.  A token may select an expert
 * more than once (each slot counts).  latent, inter: multiples of 32, at most
 * 4096; T * top_k <= 1024; top_k <= 32; n_experts <= 1024.
 * ws: k2_moe_workspace_bytes(T, top_k, latent, inter) bytes, 256-byte
 * aligned.  The result does not depend on timing (fixed summation order). */
size_t k2_moe_workspace_bytes(int T, int top_k, int latent, int inter);
int k2_moe_expert_gemv(const float *z, int T, int latent, int inter, const int32_t *topk_idx,
                       const float *topk_w, int top_k, int n_experts, const uint8_t *w13q,
                       const uint8_t *w13s, const uint8_t *w2q, const uint8_t *w2s, float *r,
                       int32_t *d_err, void *ws, size_t ws_bytes, void *stream);

typedef struct {
    int hidden, latent, inter, n_experts, top_k, n_shared;
    float routed_scale;
    float eps;                    /* latent RMSNorm */
} k2_moe_config;

/* Weights of one latent-MoE layer (host struct of device pointers). */
typedef struct {
    k2_moe_config cfg;
    const uint16_t *w_router;     /* bf16 [n_experts][hidden] */
    const float *router_bias;     /* fp32 [n_experts], nullable = zeros */
    const uint16_t *w_down;       /* bf16 [latent][hidden] */
    const float *latent_gamma;    /* fp32 [latent] */
    const uint16_t *w_up;         /* bf16 [hidden][latent] */
    const uint8_t *w13q, *w13s;   /* routed experts, layout of k2_moe_expert_gemv */
    const uint8_t *w2q, *w2s;
    const uint16_t *sh_w13;       /* bf16 [n_shared][2 inter][hidden]: W1 rows, then W3 rows */
    const uint16_t *sh_w2;        /* bf16 [n_shared][hidden][inter] */
} k2_moe_layer_weights;

/* The whole layer on x [T][hidden] fp32:
 *   route (k2_moe_route on x), z = RMSNorm(W_dn x) * latent_gamma (one group,
 *   eps), r = k2_moe_expert_gemv(z), y = W_up r + sum_s W2_s(silu(W1_s x) *
 *   (W3_s x)).
 * y: [T][hidden], overwritten.  topk_idx_out / topk_w_out ([T][top_k],
 * nullable) receive the routing.  d_err as in k2_moe_expert_gemv.  Limits:
 * those of k2_moe_route and k2_moe_expert_gemv.  ws:
 * k2_moe_layer_workspace_bytes(&cfg, T) bytes, 256-byte aligned.  The
 * router and the shared experts (they read only x) are forked onto a stream
 * of the library's own (one per device, created on first use, default
 * priority) after an event recorded on `stream`, which waits for the
 * routing before the routed experts and for the shared experts before W_up:
 * the call stays ordered on `stream` and can be captured into a graph from
 * it (a call captured before the device's first uncaptured call runs on
 * `stream` alone); calls that overlap in time on one device must not (they
 * would share that stream). */
size_t k2_moe_layer_workspace_bytes(const k2_moe_config *cfg, int T);
int k2_moe_layer(const k2_moe_layer_weights *w, const float *x, int T, float *y,
                 int32_t *topk_idx_out, float *topk_w_out, int32_t *d_err, void *ws,
                 size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Measurement utility (not a step of the path)
 * ---------------------------------------------------------------------- */

/* Streaming read of buf[0, bytes) split into `blocks` contiguous slabs of
 * floor(bytes / 16 / blocks) 16-byte words (one 256-thread block each), with
 * the decode GEMVs' load policy (non-temporal 128-bit loads, 8 in flight per
 * thread); the tail past blocks * slab is not read.  sink: device uint32
 * [blocks], receives one word per block.  Timing repeated launches over a
 * buffer far larger than the memory-side cache gives the read bandwidth the
 * weight stream can reach ("achievable" beside the 8 TB/s peak).  K2_EINVAL
 * for null / misaligned pointers or bytes < 16 * blocks. */
int k2_read_probe(const void *buf, size_t bytes, int blocks, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* K2_H */
