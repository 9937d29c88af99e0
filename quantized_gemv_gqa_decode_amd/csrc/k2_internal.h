// k2_internal.h -- argument blocks and launchers shared between the
// translation units of libk2 (not part of the C ABI).
#pragma once

#include "k2_dev.h"

#define K2_MAX_GROUPS 8
#define K2_MAX_LDS_FLOATS 12288          // 48 KiB of staged activations
#define K2_GEMV_MAX_BLOCKS 4096
#define K2_ATTN_MAX_CHUNK 1024           // positions per attention block
#ifndef K2_ATTN_MIN_CHUNK
#define K2_ATTN_MIN_CHUNK 64
#endif
#ifndef K2_ATTN_TARGET_BLOCKS
#define K2_ATTN_TARGET_BLOCKS 256
#endif
#define K2_ATTN_MAX_SPLITS 512           // combine LDS bound: >= max splits
#define K2_ARGMAX_MAX_BLOCKS K2_GEMV_MAX_BLOCKS

namespace k2 {

enum { PRO_NONE = 0, PRO_NORM = 1 };
enum { EPI_PLAIN = 0, EPI_SWIGLU = 1, EPI_ARGMAX = 2 };

// Cross-block argmax: every block of the producing kernel writes its
// (value, index) candidate; argmax_final_kernel reduces them in block order
// (a fixed order, so the result does not depend on timing).  The kernel
// boundary orders the two.  (A last-arriving-block reduction would need one
// device-scope atomic per block on one counter: thousands of them serialize
// to tens of microseconds, far more than a second launch.)
struct ArgmaxArgs {
    float *part_v;
    int *part_i;
    int32_t *out_idx;
    int n_blocks;
    // nullable: the final reduction also advances a device position held
    // there by one when it lies in [0, adv_cap) (the last kernel of a decode
    // step whose position is read from device memory)
    int32_t *adv_pos;
    int adv_cap;
};

struct GemvArgs {
    const void *W;
    const float *Sf;           // fp8 row scales
    const uint8_t *S8;         // MXFP4 E8M0 scales
    const float *x;            // [B][K] (or h for PRO_NORM)
    const float *gamma;        // PRO_NORM
    float eps;                 // PRO_NORM
    int groups;                // PRO_NORM
    float *y;
    const float *residual;     // nullable, [B][N]
    int N, K, B;
    int n_out;                 // EPI_SWIGLU: inter (N = 2 * inter)
    int64_t n_units;
    ArgmaxArgs am;             // EPI_ARGMAX
};

int gemv_dispatch(int wdt, const GemvArgs &a, int pro, int epi, hipStream_t st);

// ------------------------------------------------------------- attention --

struct AttnArgs {
    const float *q;            // rotated q [n_qh][hd]  (unfused)
    const float *qkv;          // raw projection (fused)
    const float *cos_sin;      // [cap][hd/2][2] (fused)
    void *kc, *vc;
    float *ks, *vs;
    float *out;                // [n_qh][hd]
    float *part;               // [n_kv][S][rep][hd]
    float *part_ml;            // [n_kv][S][rep][2]
    unsigned *head_cnt;        // [n_kv] split arrivals (zero between calls)
    unsigned *ao_sync;         // attention + O launch: AO_SYNC_WORDS (zero between calls)
    int n_qh, n_kv, cap, len, pos, chunk, S;
    float scale;
    // Position read from device memory (nullable): when set, pos, len,
    // chunk and S are derived on the device from *d_pos by the rule of
    // attn_splits, the grid covers the most splits the cache capacity
    // allows (S above is that grid extent), and blocks past the device split
    // count exit at once.  A position outside [0, cap) sets *d_err (nullable)
    // to K2_ERANGE and the launch writes nothing.
    const int32_t *d_pos;
    int32_t *d_err;
    // Weight bytes of the phase that follows (optional): blocks of the
    // launch beyond the attention grid read this range once so that it sits
    // in the memory-side cache when the next GEMV streams it.  Read only;
    // nothing is computed from it here.
    const void *pf;
    int64_t pf_bytes;
};

size_t attn_ws_bytes(int n_qh, int n_kv, int hd, int cap);
int attn_splits(int n_kv, int len, int *chunk);
int attn_max_splits(int n_kv, int cap);
int attn_launch(int kvdt, int hd, int rep, bool fused, const AttnArgs &a, hipStream_t st);
int device_cus();

// A prefill chunk's attention: RoPE and cache append of the T rows of qkv
// ([T][(n_qh + 2 n_kv) hd], positions pos0 ..), then every row's query over
// the cache up to its own position, in one launch (out [T][n_qh][hd];
// qrot [T][n_qh][hd] scratch).  ws: attn_rows_ws_bytes (split partials);
// cnt: attn_rows_cnt_bytes of split counters, zero-filled before its first
// use and left zero by every launch.  K2_EUNSUPPORTED (nothing enqueued)
// unless hd = 128 and n_qh / n_kv is 1, 2, 4 or 8.
size_t attn_rows_ws_bytes(int n_qh, int n_kv, int hd, int cap, int T);
size_t attn_rows_cnt_bytes(int n_kv, int T);
// From ATTN_PREFILL_MIN_T rows on (from ATTN_PREFILL_LONG_MIN_T rows once
// the cache holds more than ATTN_PREFILL_LONG_LEN positions), attn_rows_launch
// runs the attention of a bf16 / int8 cache through attn_prefill_launch
// (attn_prefill.hip): the causal attention of rows pos0 .. pos0+T-1 (qrot
// [T][n_qh][128], already rotated, K/V already appended) on the matrix
// cores, out [T][n_qh][128]; fewer rows take the split per-row kernel.
// Measured on 3.7B-shaped verification rounds (matrix cores against the
// per-row kernel): 2 rows 3.88 against 3.63 ms at 528 positions and 4.51
// against 4.19 at 8192; 8 rows 4.10 against 3.89 at 528 and 5.05 against
// 6.14 at 8192; 12-32 rows faster at every length measured.
constexpr int ATTN_PREFILL_MIN_T = 12;
constexpr int ATTN_PREFILL_LONG_MIN_T = 8;
constexpr int ATTN_PREFILL_LONG_LEN = 1024;
// part / part_ml / cnt (nullable): room for max_splits key splits of the T
// rows ([split][T][n_qh][hd] and [split][T][n_qh][2] floats) and one zeroed
// counter per (64-query block, kv head), left zero; with them a chunk whose
// query blocks leave compute units idle also splits its keys.  oh / ol
// (nullable): the output as bf16 hi / lo planes [T][n_qh hd] instead of out.
int attn_prefill_launch(int kvdt, const float *qrot, float *out, const void *kc, const void *vc, const float *ks,
                        const float *vs, int n_qh, int n_kv, int hd, int cap, int pos0, int T, float *part,
                        float *part_ml, int max_splits, unsigned *cnt, uint16_t *oh, uint16_t *ol,
                        hipStream_t st);
// oh / ol (nullable): where the matrix-core attention runs, its output goes
// to these bf16 hi / lo planes instead of out, and *planes (nullable) says
// whether it did.
// whether attn_rows_launch takes this chunk (else K2_EUNSUPPORTED)
bool attn_rows_ok(int kvdt, int n_qh, int n_kv, int hd, int cap, int pos0, int T);
int attn_rows_launch(int kvdt, const float *qkv, const float *cos_sin, float *qrot, float *out, void *kc,
                     void *vc, float *ks, float *vs, int n_qh, int n_kv, int hd, int cap, int pos0, int T,
                     void *ws, unsigned *cnt, hipStream_t st, uint16_t *oh = nullptr, uint16_t *ol = nullptr,
                     bool *planes = nullptr, bool appended = false);

// Sync words of the attention + O launch: the O-block counter on a line of
// its own, and 16 copies (one 256-byte line each) of the per-kv-head ready
// flags, so that the O blocks' polling spreads over memory channels.
constexpr int AO_SYNC_HEADS = 0;           // kv heads whose output is stored
constexpr int AO_SYNC_ODONE = 64;          // O blocks finished
constexpr int AO_READY_COPIES = 16;
constexpr int AO_SYNC_READY = 128;         // [copy * 64]: every head's output is stored
constexpr int AO_SYNC_WORDS = AO_SYNC_READY + AO_READY_COPIES * 64;

// Attention followed by the O projection (+ residual) in one launch when
// the shape has an instantiation and both grids fit on the chip at once;
// K2_EUNSUPPORTED otherwise (nothing enqueued).
int attn_o_launch(int wdt, int kvdt, int hd, int rep, const AttnArgs &at, const GemvArgs &o,
                  int32_t *d_err, hipStream_t st);

// Fused-form attention (at) and then the O GEMV + residual (o, B = 1): one
// launch where attn_o_launch has one and the cache is fp32 or bf16, else the
// two kernels, the attention launch's idle compute units prefetching the O
// weights.
int attn_then_o(int wdt, int kvdt, int hd, int rep, AttnArgs at, const GemvArgs &o, int32_t *d_err,
                hipStream_t st);
void attn_ws_carve(void *ws, int n_qh, int n_kv, int hd, int cap, AttnArgs &a);

// --------------------------------------------------------------- argmax --

size_t argmax_ws_bytes();
void argmax_ws_carve(void *ws, ArgmaxArgs &am);

// ------------------------------------------------------------------- misc --

int embed_launch(int embdt, const void *E, int H, int vocab, int token, const int32_t *d_token,
                 int32_t *d_err, float *h, hipStream_t st);
// GroupedRMSNorm of `rows` rows (one block per row and group)
int rmsnorm_rows_launch(const float *x, const float *gamma, float *y, int rows, int hidden, int groups,
                        float eps, hipStream_t st);
// the same norm written as bf16 hi / lo planes [rows][hidden] (hi = bf16(y),
// lo = bf16(y - hi)): the input form of gemm_mfma_planes
int rmsnorm_rows_planes_launch(const float *x, const float *gamma, uint16_t *yh, uint16_t *yl, int rows,
                               int hidden, int groups, float eps, hipStream_t st);
int argmax_final_launch(const ArgmaxArgs &am, int n_blocks, hipStream_t st);
// Advance a device position by one when it lies in [0, cap) (one thread).
int pos_advance_launch(int32_t *d_pos, int cap, hipStream_t st);

// ------------------------------------------------------ device functions --

__device__ __forceinline__ void argmax_pair_max(float &v, int &i, float ov, int oi)
{
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}

__device__ __forceinline__ void argmax_wave(float &v, int &i)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o, K2_WAVE);
        const int oi = __shfl_xor(i, o, K2_WAVE);
        argmax_pair_max(v, i, ov, oi);
    }
}

// Block-level (value, index) reduction; result valid in thread 0.
__device__ __forceinline__ void argmax_block(float &v, int &i)
{
    __shared__ float sv[K2_WAVES_PER_BLOCK];
    __shared__ int si[K2_WAVES_PER_BLOCK];
    argmax_wave(v, i);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) { sv[wave] = v; si[wave] = i; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < K2_WAVES_PER_BLOCK; ++w) argmax_pair_max(v, i, sv[w], si[w]);
    }
    __syncthreads();
}

// bf16-weight product with 2..32+ token rows on the matrix cores
// (dense_mfma.hip): y = W x for T >= 2 rows through per-split partials.
enum { DM_EPI_PLAIN = 0, DM_EPI_ADD = 1, DM_EPI_SWIGLU = 2 };
bool dense_mfma_ok(int N, int K);
size_t dense_mfma_ws_bytes(int N, int K, int T);
// A small-T product's optional grouped-RMSNorm prologue: x is the residual
// stream h and the product multiplies gamma * h / rms(group); nsq [T][K / 64]
// holds the partial sums of squares over 64 consecutive elements that the
// product which last added into h wrote through its osq (gamma null: none).
struct DmNorm {
    const float *gamma = nullptr, *nsq = nullptr;
    int groups = 1;
    float eps = 0.f;
};
bool dense_norm_ok(int hidden, int groups);
// The QKV product's optional epilogue in a prefill chunk: split-half RoPE of
// q and k (head_dim 128) at positions pos0 + t, q into qrot [T][n_qh][128],
// k and v appended to the cache (format kvdt) at those slots.  dense_mfma
// takes it only where the product's last blocks sum the partials (cnt
// given, tokens x splits small); it returns K2_EUNSUPPORTED, nothing
// enqueued, where it would not, and the caller appends separately.
struct DmRope {
    const float *cs = nullptr;                 // [cap][64][2] cos, sin
    float *qrot = nullptr;
    void *kc = nullptr, *vc = nullptr;
    float *ks = nullptr, *vs = nullptr;
    int n_qh = 0, n_kv = 0, cap = 0, pos0 = 0, kvdt = 0;
};
int dense_mfma(const uint16_t *W, const float *x, float *y, int N, int K, int T, int epi, float *part,
               hipStream_t st, unsigned *cnt = nullptr, const DmNorm &nrm = DmNorm{}, float *osq = nullptr,
               const DmRope *rope = nullptr);
int dense_mfma_cnt_words(int N);

// The projections of a prefill chunk of 1..GM_MAX_T positions on the matrix
// cores (gemm_mfma.hip): y [T][N] = x [T][K] W^T with the epilogue epi
// (SwiGLU: y [T][N/2], gate rows n, up rows n + N/2), W of format wdt
// (K2_BF16, K2_FP8E4M3, K2_MXFP4, K2_Q4S) with its scales Ws as in a
// k2_layer.  ws: gemm_mfma_ws_bytes (the activation planes and split
// partials; no state kept between calls).  K2_EUNSUPPORTED (nothing
// enqueued) unless K % 128 == 0 and N % 4 == 0 (SwiGLU: N % 256 == 0).
constexpr int GM_MAX_T = 256;
bool gemm_mfma_ok(int N, int K, int epi);
size_t gemm_mfma_ws_bytes(int wdt, int N, int K, int T, int epi);
int gemm_mfma(int wdt, const void *W, const void *Ws, const float *x, float *y, int N, int K, int T, int epi,
              void *ws, hipStream_t st);
// The same product with the activations given as bf16 hi / lo planes
// [gemm_mfma_rows(T, wdt)][K] (rows past T may hold anything), and for
// SwiGLU optionally its output written as planes yh / yl [T][N/2] instead
// of y: the forms the producers of a prefill chunk's activations write.
int gemm_mfma_planes(int wdt, const void *W, const void *Ws, const uint16_t *xh, const uint16_t *xl, float *y,
                     uint16_t *yh, uint16_t *yl, int N, int K, int T, int epi, void *ws, hipStream_t st);
int gemm_mfma_rows(int T, int wdt);

}  // namespace k2
