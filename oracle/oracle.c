/*
 * oracle.c -- plain, slow, fp64 CPU reference of the batch-1 decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library; the product path never does.  It shares
 * no source, header, table or helper with the HIP library: every codec and
 * every step below is written out here from its definition.
 *
 * Sources (page titles as they appear in the reference pages):
 *   [k2-burn]   README of k2-burn (K2-Horizon port): "Model shape",
 *               "Working end to end" (GroupedRMSNorm, split-half RoPE, GQA,
 *               SwiGLU), "KV cache storage" (symmetric int8 + per-head_dim
 *               block scale), "Quantization" (fp8 E4M3 for Linear weights).
 *   [k3_run.c]  kimi-k3-in-c, src/cli/k3_run.c: header comment (experts
 *               "multiplied straight out of MXFP4"), real_cfg_hardcoded()
 *               (latent MoE: 896 experts, top-16, 2 shared, latent 3584,
 *               inter 3072, routed_scale 1.0, renorm, latent_norm), argmax_()
 *               (first maximum wins).
 *   [cpu_weights.rs] avarok_core kimi_k3 cpu_weights.rs: MoeWeights layout
 *               (down, up, norm, router, bias, experts (w1, w2, w3), shared).
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 * Arithmetic is fp64 except the storage roundings the method defines (weight
 * quantizers, KV-cache store), which are done in fp32 exactly as defined.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_EXPORT __attribute__((visibility("default")))

/* dtype tags used by the oracle's own structs */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_MXFP4 = 3, ORC_I8 = 4, ORC_Q4S = 5 };

/* ------------------------------------------------------------------------ */
/* Storage codecs                                                            */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16: the upper 16 bits of an IEEE binary32. */
ORC_EXPORT double orc_bf16_value(uint16_t b) { return (double)f32_from_bits((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). The value is
 * chosen as the nearer of the two bf16 neighbours by exact comparison in
 * fp64; on a tie the one with an even last mantissa bit wins. */
ORC_EXPORT uint16_t orc_bf16_round(float x)
{
    uint32_t u = bits_from_f32(x);
    uint16_t lo = (uint16_t)(u >> 16);           /* truncation toward zero */
    if ((u & 0xFFFFu) == 0) return lo;
    uint16_t hi = (uint16_t)(lo + 1);            /* next magnitude up */
    double dlo = fabs((double)x - orc_bf16_value(lo));
    double dhi = fabs((double)x - orc_bf16_value(hi));
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) ? hi : lo;
}

/* OCP FP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite 448.  Exponent field 0 holds
 * the subnormals m/8 * 2^-6. */
ORC_EXPORT double orc_fp8_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp(m / 8.0, -6);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP E2M1 (MXFP4 element): sign bit 3, exponent bits 2..1 (bias 1),
 * mantissa bit 0; exponent 0 is the subnormal m * 0.5.  The eight magnitudes
 * are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
ORC_EXPORT double orc_e2m1_value(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E8M0 shared scale: 2^(byte - 127); 0xFF is NaN. */
ORC_EXPORT double orc_e8m0_value(uint8_t b)
{
    if (b == 255) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/*
 * Round a non-negative finite double `a` onto the grid of a small float
 * format with `mbits` mantissa bits, minimum normal exponent `emin`
 * (unbiased) and largest finite value `maxv`, to nearest with ties to even,
 * saturating at maxv.  Returns the grid value (exact in double).
 *
 * Inside binade [2^e, 2^(e+1)) (e >= emin) the grid step is 2^(e-mbits);
 * below 2^emin the step stays 2^(emin-mbits) (subnormals).  `a / step` is
 * exact in double, so nearbyint() (round-half-even under the default mode)
 * makes the decision.  A result equal to 2^(e+1) is the next binade's first
 * value and needs no fix-up.
 */
static double round_to_grid(double a, int mbits, int emin, double maxv)
{
    if (a >= maxv) return maxv;
    int e;
    if (a < ldexp(1.0, emin)) e = emin;
    else { frexp(a, &e); e -= 1; }              /* a in [2^e, 2^(e+1)) */
    double step = ldexp(1.0, e - mbits);
    double q = nearbyint(a / step) * step;
    return q > maxv ? maxv : q;
}

/* fp32 -> E4M3FN code, RNE, saturating at +-448.  The sign of the input is
 * kept (so -0.0 and small negatives give 0x80). */
ORC_EXPORT uint8_t orc_fp8_encode(float x)
{
    int neg = signbit(x) != 0;
    double g = round_to_grid(fabs((double)x), 3, -6, 448.0);
    /* find the code whose value is g: scan the 127 finite magnitudes */
    for (int c = 0; c < 127; ++c)
        if (orc_fp8_value((uint8_t)c) == g) return (uint8_t)(c | (neg ? 0x80 : 0));
    return 0x7F; /* unreachable for finite input */
}

/* fp32 -> E2M1 code (4 bits), RNE, saturating at +-6; sign kept. */
ORC_EXPORT uint8_t orc_e2m1_encode(float x)
{
    int neg = signbit(x) != 0;
    double g = round_to_grid(fabs((double)x), 1, 0, 6.0);
    for (int c = 0; c < 8; ++c)
        if (orc_e2m1_value((uint8_t)c) == g) return (uint8_t)(c | (neg ? 8 : 0));
    return 7;
}

/*
 * fp8 weight quantizer ("--scheme fp8", [k2-burn] "Quantization"; per-output
 * row fp32 scale).  Reading taken: s_n = fp32(amax_n / 448) with IEEE fp32
 * division, code = E4M3FN-RNE-saturate(fp32(w / s_n)); an all-zero row gets
 * s_n = 0 and codes 0.  Dequantized weight = dec(code) * s_n.
 * w: bf16 bits [N][K] (the bf16 draw is the quantizer's input).
 */
ORC_EXPORT void orc_quant_fp8_rows(const uint16_t *w, int64_t N, int64_t K,
                                   uint8_t *codes, float *scale)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = w + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(f32_from_bits((uint32_t)row[k] << 16));
            if (a > amax) amax = a;
        }
        volatile float s = amax / 448.0f;       /* one fp32 division */
        scale[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            if (amax == 0.0f) { codes[n * K + k] = 0; continue; }
            volatile float t = f32_from_bits((uint32_t)row[k] << 16) / s;
            codes[n * K + k] = orc_fp8_encode(t);
        }
    }
}

/*
 * MXFP4 quantizer (OCP Microscaling v1.0 reading; element E2M1, block 32,
 * shared scale E8M0).  Per row, per block of 32 consecutive k:
 *   E   = unbiased exponent field of fp32 amax (field - 127; a zero or
 *         subnormal amax has field 0, so E = -127),
 *   e_b = clamp(E - 2, -127, 127)   (2 = largest E2M1 exponent),
 *   byte = e_b + 127,
 *   code = E2M1-RNE-saturate(w * 2^-e_b)  (exact power-of-two scaling).
 * Packing: q[n][k/2], low nibble = even k, high nibble = odd k;
 *          e[n][k/32].
 */
ORC_EXPORT void orc_quant_mxfp4(const uint16_t *w, int64_t N, int64_t K,
                                uint8_t *q, uint8_t *e)
{
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *blk = w + n * K + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(f32_from_bits((uint32_t)blk[i] << 16));
                if (a > amax) amax = a;
            }
            int E = (int)((bits_from_f32(amax) >> 23) & 0xFF) - 127;
            int eb = E - 2;
            if (eb < -127) eb = -127;
            if (eb > 127) eb = 127;
            e[n * nb + b] = (uint8_t)(eb + 127);
            for (int i = 0; i < 32; i += 2) {
                float x0 = (float)ldexp((double)f32_from_bits((uint32_t)blk[i] << 16), -eb);
                float x1 = (float)ldexp((double)f32_from_bits((uint32_t)blk[i + 1] << 16), -eb);
                uint8_t c0 = orc_e2m1_encode(x0), c1 = orc_e2m1_encode(x1);
                q[n * (K / 2) + b * 16 + i / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/*
 * Q4S weights ([k2-burn] "Working end to end" and "Quantization": the
 * quantizer writes int4 "Q4S" checkpoints, block size 64).  The pages name
 * nothing more; reading taken: symmetric signed int4 on [-7, 7] (the S of
 * Q4S; two's complement nibbles, -8 never produced) with one fp32 scale per
 * 64 consecutive k of a row, built like the int8 KV codec:
 *   a = max|w| over the block, s = fp32(a / 7),
 *   code = clamp(rint(fp32(w / s)), -7, 7)   (ties to even),
 *   a = 0 gives s = 0 and codes 0;  value = code * s.
 * Packing: q[n][k/2], low nibble = even k, high nibble = odd k; s[n][k/64].
 */
ORC_EXPORT double orc_q4s_value(uint8_t nib)
{
    nib &= 15;
    return (double)((nib & 8) ? (int)nib - 16 : (int)nib);
}

ORC_EXPORT void orc_quant_q4s(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s)
{
    const int64_t nb = K / 64;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *blk = w + n * K + b * 64;
            float amax = 0.0f;
            for (int i = 0; i < 64; ++i) {
                float a = fabsf(f32_from_bits((uint32_t)blk[i] << 16));
                if (a > amax) amax = a;
            }
            volatile float sc = amax / 7.0f;
            s[n * nb + b] = amax == 0.0f ? 0.0f : sc;
            for (int i = 0; i < 64; i += 2) {
                int c[2] = {0, 0};
                for (int j = 0; j < 2 && amax != 0.0f; ++j) {
                    volatile float t = f32_from_bits((uint32_t)blk[i + j] << 16) / sc;
                    double r = nearbyint((double)t);
                    if (r > 7) r = 7;
                    if (r < -7) r = -7;
                    c[j] = (int)r;
                }
                q[n * (K / 2) + b * 32 + i / 2] = (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
            }
        }
    }
}

/*
 * int8 KV-cache codec ([k2-burn] "KV cache storage": symmetric int8 with a
 * scale per head_dim block).  Reading taken: a = max|x| over the block,
 * s = fp32(a / 127), code = clamp(rint(fp32(x / s)), -127, 127) (ties to
 * even); a = 0 gives s = 0 and codes 0.  Dequantized value = fp32(code * s).
 */
ORC_EXPORT void orc_kv_quant_int8(const float *x, int n, int8_t *codes, float *scale)
{
    float a = 0.0f;
    for (int i = 0; i < n; ++i) { float t = fabsf(x[i]); if (t > a) a = t; }
    if (a == 0.0f) {
        *scale = 0.0f;
        for (int i = 0; i < n; ++i) codes[i] = 0;
        return;
    }
    volatile float s = a / 127.0f;
    *scale = s;
    for (int i = 0; i < n; ++i) {
        volatile float t = x[i] / s;
        double r = nearbyint((double)t);
        if (r > 127) r = 127;
        if (r < -127) r = -127;
        codes[i] = (int8_t)r;
    }
}

ORC_EXPORT double orc_int8_dequant(int8_t code, float scale)
{
    volatile float v = (float)code * scale;   /* fp32(code * s) */
    return (double)v;
}

/* ------------------------------------------------------------------------ */
/* Weight matrices: y = W_hat x in fp64                                      */
/* ------------------------------------------------------------------------ */

/* A projection matrix in storage format, row-major [N][K].
 *   F32:   w = float[N][K]
 *   BF16:  w = uint16[N][K]
 *   FP8:   w = uint8 codes [N][K], s = float row scale [N]
 *   MXFP4: w = uint8 [N][K/2] (low nibble even k), s = uint8 E8M0 [N][K/32]
 *   Q4S:   w = uint8 [N][K/2] (low nibble even k), s = float [N][K/64] */
typedef struct {
    int dtype;
    const void *w;
    const void *s;
} orc_mat;

static double row_dot(const orc_mat *m, int64_t n, int64_t K, const double *x)
{
    double acc = 0.0;
    switch (m->dtype) {
    case ORC_F32: {
        const float *r = (const float *)m->w + n * K;
        for (int64_t k = 0; k < K; ++k) acc += (double)r[k] * x[k];
        return acc;
    }
    case ORC_BF16: {
        const uint16_t *r = (const uint16_t *)m->w + n * K;
        for (int64_t k = 0; k < K; ++k) acc += orc_bf16_value(r[k]) * x[k];
        return acc;
    }
    case ORC_FP8: {
        const uint8_t *r = (const uint8_t *)m->w + n * K;
        for (int64_t k = 0; k < K; ++k) acc += orc_fp8_value(r[k]) * x[k];
        return acc * (double)((const float *)m->s)[n];
    }
    case ORC_MXFP4: {
        const uint8_t *r = (const uint8_t *)m->w + n * (K / 2);
        const uint8_t *sc = (const uint8_t *)m->s + n * (K / 32);
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = r[k / 2];
            uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
            acc += orc_e2m1_value(nib) * orc_e8m0_value(sc[k / 32]) * x[k];
        }
        return acc;
    }
    case ORC_Q4S: {
        const uint8_t *r = (const uint8_t *)m->w + n * (K / 2);
        const float *sc = (const float *)m->s + n * (K / 64);
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = r[k / 2];
            uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
            acc += orc_q4s_value(nib) * (double)sc[k / 64] * x[k];
        }
        return acc;
    }
    }
    return NAN;
}

ORC_EXPORT void orc_matvec(int dtype, const void *w, const void *s, const double *x,
                           double *y, int64_t N, int64_t K)
{
    orc_mat m = { dtype, w, s };
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) y[n] = row_dot(&m, n, K, x);
}

/* ------------------------------------------------------------------------ */
/* Norm, RoPE, attention, activation                                         */
/* ------------------------------------------------------------------------ */

/* GroupedRMSNorm ([k2-burn] "Model shape": layernorm_num_groups=2).
 * Reading taken: the hidden vector is cut into G equal contiguous groups; each
 * group is divided by sqrt(mean of its squares + eps); the gain is applied
 * elementwise over the full hidden size. */
ORC_EXPORT void orc_rmsnorm_grouped(const double *h, const float *gamma, double *y,
                                    int H, int G, double eps)
{
    int gs = H / G;
    for (int g = 0; g < G; ++g) {
        double ss = 0.0;
        for (int i = 0; i < gs; ++i) ss += h[g * gs + i] * h[g * gs + i];
        double r = 1.0 / sqrt(ss / gs + eps);
        for (int i = 0; i < gs; ++i) y[g * gs + i] = h[g * gs + i] * r * (double)gamma[g * gs + i];
    }
}

/* Split-half rotary embedding ([k2-burn] "Working end to end": split-half
 * RoPE; default rope type).  Within a head of size hd, element i pairs with
 * i + hd/2 and the pair is rotated by angle pos * theta^(-2i/hd):
 *   u_i       <- a cos - b sin
 *   u_{i+hd/2} <- a sin + b cos. */
ORC_EXPORT void orc_rope(double *u, int n_heads, int hd, int pos, double theta)
{
    int half = hd / 2;
    for (int h = 0; h < n_heads; ++h) {
        double *v = u + (int64_t)h * hd;
        for (int i = 0; i < half; ++i) {
            double ang = (double)pos * pow(theta, -2.0 * i / hd);
            double c = cos(ang), s = sin(ang);
            double a = v[i], b = v[i + half];
            v[i] = a * c - b * s;
            v[i + half] = a * s + b * c;
        }
    }
}

ORC_EXPORT double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* One KV-cache slot in storage format: cache [n_kv][cap][hd] of dtype kvdt,
 * int8 scales [n_kv][cap]. */
static double kv_read(int kvdt, const void *c, const float *sc, int64_t idx, int64_t sidx)
{
    switch (kvdt) {
    case ORC_F32: return (double)((const float *)c)[idx];
    case ORC_BF16: return orc_bf16_value(((const uint16_t *)c)[idx]);
    case ORC_I8: return orc_int8_dequant(((const int8_t *)c)[idx], sc[sidx]);
    }
    return NAN;
}

/* Store the fp64 vector u (one kv head, hd values) at slot `pos`: the value
 * is first rounded to fp32 (what an fp32 pipeline holds), then stored as fp32,
 * bf16 (RNE) or int8 (block codec above). */
ORC_EXPORT void orc_kv_store(int kvdt, const double *u, void *c, float *sc, int n_kv,
                             int hd, int cap, int pos)
{
    float tmp[1024];
    int8_t q[1024];
    for (int g = 0; g < n_kv; ++g) {
        int64_t base = ((int64_t)g * cap + pos) * hd;
        for (int d = 0; d < hd; ++d) tmp[d] = (float)u[(int64_t)g * hd + d];
        if (kvdt == ORC_F32) {
            for (int d = 0; d < hd; ++d) ((float *)c)[base + d] = tmp[d];
        } else if (kvdt == ORC_BF16) {
            for (int d = 0; d < hd; ++d) ((uint16_t *)c)[base + d] = orc_bf16_round(tmp[d]);
        } else {
            float s;
            orc_kv_quant_int8(tmp, hd, q, &s);
            for (int d = 0; d < hd; ++d) ((int8_t *)c)[base + d] = q[d];
            sc[(int64_t)g * cap + pos] = s;
        }
    }
}

/* GQA decode attention for one new query position over cache slots
 * [0, len); query heads are independent (OpenMP over heads).  Query head h reads kv head floor(h / (n_qh / n_kv)) (contiguous
 * groups: the 4x repeat of [k2-burn] "Model shape").  Scores are scaled by
 * 1/sqrt(hd); the softmax subtracts the row maximum; all in fp64.
 * probs (nullable) receives [n_qh][len]. */
ORC_EXPORT void orc_attention(int kvdt, const double *q, const void *kc, const void *vc,
                              const float *ks, const float *vs, double *out, int n_qh,
                              int n_kv, int hd, int cap, int len, double *probs)
{
    int rep = n_qh / n_kv;
    double scale = 1.0 / sqrt((double)hd);
    #pragma omp parallel for schedule(static)
    for (int h = 0; h < n_qh; ++h) {
        double *s = (double *)malloc(sizeof(double) * (size_t)len);
        int g = h / rep;
        const double *qh = q + (int64_t)h * hd;
        double mx = -INFINITY;
        for (int j = 0; j < len; ++j) {
            double acc = 0.0;
            int64_t base = ((int64_t)g * cap + j) * hd;
            for (int d = 0; d < hd; ++d)
                acc += qh[d] * kv_read(kvdt, kc, ks, base + d, (int64_t)g * cap + j);
            s[j] = acc * scale;
            if (s[j] > mx) mx = s[j];
        }
        double sum = 0.0;
        for (int j = 0; j < len; ++j) { s[j] = exp(s[j] - mx); sum += s[j]; }
        for (int j = 0; j < len; ++j) s[j] /= sum;
        if (probs) for (int j = 0; j < len; ++j) probs[(int64_t)h * len + j] = s[j];
        double *oh = out + (int64_t)h * hd;
        for (int d = 0; d < hd; ++d) oh[d] = 0.0;
        for (int j = 0; j < len; ++j) {
            int64_t base = ((int64_t)g * cap + j) * hd;
            for (int d = 0; d < hd; ++d)
                oh[d] += s[j] * kv_read(kvdt, vc, vs, base + d, (int64_t)g * cap + j);
        }
        free(s);
    }
}

/* argmax with the first maximum winning ([k3_run.c] argmax_(): a later entry
 * replaces the best only when strictly greater). */
ORC_EXPORT int64_t orc_argmax(const double *v, int64_t n)
{
    int64_t b = 0;
    for (int64_t i = 1; i < n; ++i) if (v[i] > v[b]) b = i;
    return b;
}

/* ------------------------------------------------------------------------ */
/* Dense decoder step                                                        */
/* ------------------------------------------------------------------------ */

typedef struct {
    int hidden, n_layers, n_qh, n_kv, head_dim, inter, vocab, groups, cap;
    int kvdt, embdt;
    double eps, theta;
} orc_cfg;

typedef struct {
    orc_mat qkv, o, gu, down;       /* [q;k;v] rows, o, [gate;up] rows, down */
    const float *g_in, *g_post;
    void *kc, *vc;                  /* [n_kv][cap][hd] */
    float *ks, *vs;                 /* [n_kv][cap] (int8 only) */
} orc_layer;

typedef struct {
    orc_cfg cfg;
    const void *embed;              /* [vocab][hidden], fp32 or bf16 */
    orc_mat lm;                     /* [vocab][hidden] */
    const float *g_final;
    const orc_layer *layers;
} orc_model;

/*
 * One decode step for token `token` at position `pos` (0-based): the
 * pre-norm decoder layer of [k2-burn] (norm + attention residual, norm + MLP
 * residual), embed -> layers -> final norm -> untied lm_head.  The new k and v
 * are stored at slot `pos` before attending, so the token attends to itself.
 * Writes logits (nullable; when NULL the final norm and lm_head are skipped)
 * and returns the argmax (or -1 when logits is NULL).
 */
ORC_EXPORT int64_t orc_decode_step(const orc_model *m, int token, int pos, double *logits)
{
    const orc_cfg *c = &m->cfg;
    const int H = c->hidden, hd = c->head_dim, nq = c->n_qh, nkv = c->n_kv, I = c->inter;
    const int qkvn = (nq + 2 * nkv) * hd;
    double *h = calloc((size_t)H, sizeof(double));
    double *x = calloc((size_t)H, sizeof(double));
    double *qkv = calloc((size_t)qkvn, sizeof(double));
    double *o = calloc((size_t)nq * hd, sizeof(double));
    double *t = calloc((size_t)H, sizeof(double));
    double *gu = calloc((size_t)2 * I, sizeof(double));
    double *act = calloc((size_t)I, sizeof(double));

    for (int i = 0; i < H; ++i)
        h[i] = c->embdt == ORC_F32 ? (double)((const float *)m->embed)[(int64_t)token * H + i]
                                   : orc_bf16_value(((const uint16_t *)m->embed)[(int64_t)token * H + i]);

    for (int l = 0; l < c->n_layers; ++l) {
        const orc_layer *L = &m->layers[l];
        orc_rmsnorm_grouped(h, L->g_in, x, H, c->groups, c->eps);
        orc_matvec(L->qkv.dtype, L->qkv.w, L->qkv.s, x, qkv, qkvn, H);
        double *q = qkv, *k = qkv + (int64_t)nq * hd, *v = k + (int64_t)nkv * hd;
        orc_rope(q, nq, hd, pos, c->theta);
        orc_rope(k, nkv, hd, pos, c->theta);
        orc_kv_store(c->kvdt, k, L->kc, L->ks, nkv, hd, c->cap, pos);
        orc_kv_store(c->kvdt, v, L->vc, L->vs, nkv, hd, c->cap, pos);
        orc_attention(c->kvdt, q, L->kc, L->vc, L->ks, L->vs, o, nq, nkv, hd, c->cap, pos + 1, NULL);
        orc_matvec(L->o.dtype, L->o.w, L->o.s, o, t, H, (int64_t)nq * hd);
        for (int i = 0; i < H; ++i) h[i] += t[i];
        orc_rmsnorm_grouped(h, L->g_post, x, H, c->groups, c->eps);
        orc_matvec(L->gu.dtype, L->gu.w, L->gu.s, x, gu, 2 * I, H);
        for (int i = 0; i < I; ++i) act[i] = orc_silu(gu[i]) * gu[I + i];
        orc_matvec(L->down.dtype, L->down.w, L->down.s, act, t, H, I);
        for (int i = 0; i < H; ++i) h[i] += t[i];
    }
    int64_t next = -1;
    if (logits) {
        orc_rmsnorm_grouped(h, m->g_final, x, H, c->groups, c->eps);
        orc_matvec(m->lm.dtype, m->lm.w, m->lm.s, x, logits, c->vocab, H);
        next = orc_argmax(logits, c->vocab);
    }
    free(h); free(x); free(qkv); free(o); free(t); free(gu); free(act);
    return next;
}

/* ------------------------------------------------------------------------ */
/* Latent-MoE layer ([k3_run.c] real_cfg_hardcoded, [cpu_weights.rs]         */
/* MoeWeights)                                                               */
/* ------------------------------------------------------------------------ */

/*
 * Router for one token: sigma = sigmoid(W_r x); the top-k experts by
 * sigma + bias (bias used for selection only), ordered by descending score
 * with the lower expert index first on equal scores; gate
 * g_e = routed_scale * sigma_e / sum over the selected sigma (renormalised).
 * W_r: [n_experts][hidden] in storage format.
 */
ORC_EXPORT void orc_moe_route(const orc_mat *wr, const float *bias, const double *x, int hidden,
                              int n_experts, int top_k, double routed_scale, int32_t *sel,
                              double *gate)
{
    double *sig = malloc(sizeof(double) * (size_t)n_experts);
    double *score = malloc(sizeof(double) * (size_t)n_experts);
    char *taken = calloc((size_t)n_experts, 1);
    orc_matvec(wr->dtype, wr->w, wr->s, x, sig, n_experts, hidden);
    for (int e = 0; e < n_experts; ++e) {
        sig[e] = 1.0 / (1.0 + exp(-sig[e]));
        score[e] = sig[e] + (double)bias[e];
    }
    double tot = 0.0;
    for (int j = 0; j < top_k; ++j) {
        int best = -1;
        for (int e = 0; e < n_experts; ++e)
            if (!taken[e] && (best < 0 || score[e] > score[best])) best = e;
        taken[best] = 1;
        sel[j] = best;
        tot += sig[best];
    }
    for (int j = 0; j < top_k; ++j) gate[j] = routed_scale * sig[sel[j]] / tot;
    free(sig); free(score); free(taken);
}

/* One SwiGLU expert: out = W2 (silu(W1 u) * (W3 u)) where W13 stacks the W1
 * (gate) rows then the W3 (up) rows, [2*inter][in]; W2 is [in_out][inter]. */
ORC_EXPORT void orc_swiglu_expert(const orc_mat *w13, const orc_mat *w2, const double *u,
                                  int in, int inter, int out_dim, double *out)
{
    double *gu = malloc(sizeof(double) * 2 * (size_t)inter);
    double *a = malloc(sizeof(double) * (size_t)inter);
    orc_matvec(w13->dtype, w13->w, w13->s, u, gu, 2 * inter, in);
    for (int i = 0; i < inter; ++i) a[i] = orc_silu(gu[i]) * gu[inter + i];
    orc_matvec(w2->dtype, w2->w, w2->s, a, out, out_dim, inter);
    free(gu); free(a);
}

/*
 * Latent-MoE layer for one token row x [hidden]:
 *   z = RMSNorm(W_dn x) over the latent (gain ones, eps),
 *   r = sum_j gate_j * Expert_{sel_j}(z),
 *   y = W_up r + sum_s Shared_s(x).
 * Routing (sel, gate) is an input here so that a caller can pass either the
 * oracle's own routing or any other fixed selection.  Expert tables are
 * indexed by expert id; only the selected entries are read.
 */
ORC_EXPORT void orc_moe_apply(const orc_mat *wdn, const orc_mat *wup, const orc_mat *ex13,
                              const orc_mat *ex2, const orc_mat *sh13, const orc_mat *sh2,
                              int n_shared, const double *x, int hidden, int latent, int inter,
                              double eps, const int32_t *sel, const double *gate, int top_k,
                              double *y)
{
    double *zr = malloc(sizeof(double) * (size_t)latent);
    double *z = malloc(sizeof(double) * (size_t)latent);
    double *r = calloc((size_t)latent, sizeof(double));
    double *t = malloc(sizeof(double) * (size_t)(latent > hidden ? latent : hidden));
    float *ones = malloc(sizeof(float) * (size_t)latent);
    for (int i = 0; i < latent; ++i) ones[i] = 1.0f;
    orc_matvec(wdn->dtype, wdn->w, wdn->s, x, zr, latent, hidden);
    orc_rmsnorm_grouped(zr, ones, z, latent, 1, eps);
    for (int j = 0; j < top_k; ++j) {
        int e = sel[j];
        orc_swiglu_expert(&ex13[e], &ex2[e], z, latent, inter, latent, t);
        for (int i = 0; i < latent; ++i) r[i] += gate[j] * t[i];
    }
    orc_matvec(wup->dtype, wup->w, wup->s, r, y, hidden, latent);
    for (int s = 0; s < n_shared; ++s) {
        orc_swiglu_expert(&sh13[s], &sh2[s], x, hidden, inter, hidden, t);
        for (int i = 0; i < hidden; ++i) y[i] += t[i];
    }
    free(zr); free(z); free(r); free(t); free(ones);
}

ORC_EXPORT int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
