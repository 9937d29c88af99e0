// gemm_mfma.hip -- Y = X W^T for a prompt chunk of up to 256 positions on
// the matrix cores: the projections of chunked prefill.
//
// [k2-burn] "Working end to end" names prefill beside single-token decode.
// With T positions at once a projection is a dense contraction ([N][K]
// weights times [K][T] activations), run here on v_mfma_f32_16x16x32_bf16.
// The weights are exact in bf16; every fp32 activation is split once into
// bf16 hi + bf16 lo (x - hi, rounded again) and both planes are multiplied,
// so ~16 bits of every activation enter an fp32 accumulation (the precision
// of dense_mfma.hip, the small-T product).
//
// Tiling: a block (4 waves) owns 256 weight rows x BT (32, 64 or 128)
// tokens and streams its k-range in chunks of 128; a wave holds 4 row tiles
// of 16 rows x BT/16 token tiles of accumulators.  Per chunk the block copies the chunk's
// activation tile (both planes) into LDS with LDS-DMA (global_load_lds) one
// chunk ahead (two LDS buffers), and every wave loads its own weight rows one
// chunk ahead into registers; an activation fragment read from LDS feeds 4
// row tiles.  In LDS a token's row of 16 16-byte k-chunks is rotated by the
// token index, so the 16 lanes that read one k-chunk of 16 consecutive
// tokens hit 16 different bank groups.
//
// The token blocks of one row block are consecutive blocks of one XCD (the
// hardware deals consecutive block ids round-robin over the 8 XCDs, and the
// block id is remapped so that they land together): they run at the same
// time and read the same weight bytes, the first from HBM and the others
// from that XCD's L2.  Short matrices split K over several blocks, whose
// partials [split][token][row] a second kernel sums in split order (a fixed
// order: deterministic) and finishes with the epilogue.  Without a split
// the epilogue runs in registers: a lane holds 4 consecutive rows of one
// token, stored as one float4 -- plain, added into y (residual), or SwiGLU,
// for which a wave's row tiles 0-1 are gate rows and 2-3 the matching up
// rows (a block then yields 128 outputs).
// MFMA operand layout (16x16x32 bf16): lane l holds A row l % 16 and B
// column l % 16, elements k = 8 (l / 16) + [0, 8); D holds column l % 16,
// rows 4 (l / 16) + [0, 4).
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

typedef short gm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gm_f32x4 __attribute__((ext_vector_type(4)));

constexpr int GM_RT = 4;                   // row tiles per wave
constexpr int GM_BM = 4 * GM_RT * 16;      // weight rows per block (256)
constexpr int GM_BK = 128;                 // k per chunk (16 k-chunks of 8)
constexpr int GM_ROWB = GM_BK * 2;         // bytes of one token's chunk row in LDS


struct GemmArgs {
    const uint16_t *W;         // [N][K] bf16
    const uint16_t *xh, *xl;   // [TP][K] bf16 planes (rows >= T zero)
    float *y;                  // [T][N] (SwiGLU: [T][N/2])
    float *part;               // [S][TP][N] when S > 1
    int N, K, T, TP, S, KS, epi, rb, tb, xcd;
};

// x [T][K] fp32 -> hi / lo bf16 planes [TP][K], rows T .. TP-1 zero
__global__ __launch_bounds__(256) void gm_split_kernel(const float *x, uint16_t *xh, uint16_t *xl, int T,
                                                       int TP, int K)
{
    const int64_t n = (int64_t)TP * K / 4;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i * 4;
        const int t = (int)(e / K);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < T) v = *reinterpret_cast<const float4 *>(x + e);
        const float f[4] = {v.x, v.y, v.z, v.w};
        uint16_t h[4], l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = f32_to_bf16_rne(f[j]);
            l[j] = f32_to_bf16_rne(f[j] - bf16_to_f32(h[j]));
        }
        uint2 hv, lv;
        hv.x = h[0] | ((uint32_t)h[1] << 16);
        hv.y = h[2] | ((uint32_t)h[3] << 16);
        lv.x = l[0] | ((uint32_t)l[1] << 16);
        lv.y = l[2] | ((uint32_t)l[3] << 16);
        *reinterpret_cast<uint2 *>(xh + e) = hv;
        *reinterpret_cast<uint2 *>(xl + e) = lv;
    }
}

// weight row of row tile rt, tile row r (0..15) of wave w in row block b
__device__ __forceinline__ int gm_row(const GemmArgs &a, int b, int w, int rt, int r)
{
    if (a.epi == DM_EPI_SWIGLU) {
        const int o = b * (GM_BM / 2) + w * 32 + (rt & 1) * 16 + r;
        return rt < 2 ? o : a.N / 2 + o;
    }
    return b * GM_BM + w * 64 + rt * 16 + r;
}

template <int BT>
__global__ __launch_bounds__(256, BT <= 64 ? 2 : 1) void gm_kernel(const GemmArgs a)
{
    constexpr int NT = BT / 16;                           // token tiles
    constexpr int PLANE = BT * GM_ROWB;                   // bytes of one plane's chunk tile
    constexpr int STAGE = 2 * PLANE;                      // hi + lo
    constexpr int NDMA = PLANE / 1024 / 4;                // 1 KiB wave copies per wave, plane and chunk
    extern __shared__ float4 lds4[];
    char *lds = reinterpret_cast<char *>(lds4);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, c16 = lane & 15;

    // block id -> (token block, row block, split), the token blocks of a row
    // block consecutive on one XCD
    const int nblk = gridDim.x;
    const int L = a.xcd ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
    const int tblk = L % a.tb, rest = L / a.tb;
    const int rb = rest % a.rb, split = rest / a.rb;
    const int t0 = tblk * BT, kbeg = split * a.KS, nch = a.KS / GM_BK;

    // this wave's row tiles; rows past N read row N-1 and are never stored
    const uint16_t *wrow[GM_RT];
#pragma unroll
    for (int rt = 0; rt < GM_RT; ++rt) {
        int r = gm_row(a, rb, wave, rt, c16);
        r = r < a.N ? r : a.N - 1;
        wrow[rt] = a.W + (int64_t)r * a.K + kbeg + q * 8;
    }
    // chunk c, k-step j of row tile rt: the 16 B at column c*128 + 32j + 8q
    // (the 4 lanes of a row read 64 contiguous bytes per instruction)
    auto load_w = [&](int c, k2_u4 (&w)[GM_RT][4]) {
#pragma unroll
        for (int rt = 0; rt < GM_RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[rt][j] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(wrow[rt] + c * GM_BK + 32 * j));
    };
    // the activation tile of chunk c into LDS buffer c & 1: wave copy i of a
    // plane covers tile bytes [(4i + wave) * 1024, + 1024); tile byte o is
    // token o / 256, slot (o % 256) / 16, and slot s of token t holds k-chunk
    // (s + t) % 16
    auto dma_x = [&](int c) {
        char *st = lds + (c & 1) * STAGE;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int o = (i * 4 + wave) * 1024 + lane * 16;
            const int t = o / GM_ROWB, slot = (o % GM_ROWB) / 16;
            const int kc = (slot + t) & 15;
            const int64_t src = (int64_t)(t0 + t) * a.K + kbeg + c * GM_BK + kc * 8;
            __builtin_amdgcn_global_load_lds(a.xh + src, st + (i * 4 + wave) * 1024, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(a.xl + src, st + PLANE + (i * 4 + wave) * 1024, 16, 0, 0);
        }
    };

    gm_f32x4 acc[GM_RT][NT];
#pragma unroll
    for (int rt = 0; rt < GM_RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[rt][tt] = gm_f32x4{0.f, 0.f, 0.f, 0.f};

    k2_u4 wc[GM_RT][4], wn[GM_RT][4];
    load_w(0, wc);
    dma_x(0);
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        __builtin_amdgcn_s_waitcnt(0);                    // this wave's copies of chunk c and its weights are in
        __syncthreads();                                  // every wave's; nobody still reads buffer (c + 1) & 1
        if (c + 1 < nch) {
            dma_x(c + 1);
            load_w(c + 1, wn);
        }
        const char *st = lds + (c & 1) * STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kc = j * 4 + q;                     // this lane's k-chunk in k-step j
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = tt * 16 + c16;
                const int off = t * GM_ROWB + ((kc - t) & 15) * 16;
                const gm_bf16x8 bh = *reinterpret_cast<const gm_bf16x8 *>(st + off);
                const gm_bf16x8 bl = *reinterpret_cast<const gm_bf16x8 *>(st + PLANE + off);
                // the hi products of all row tiles, then the lo ones: 4
                // independent MFMAs between two into one accumulator
#pragma unroll
                for (int rt = 0; rt < GM_RT; ++rt)
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gm_bf16x8, wc[rt][j]), bh,
                                                                          acc[rt][tt], 0, 0, 0);
#pragma unroll
                for (int rt = 0; rt < GM_RT; ++rt)
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gm_bf16x8, wc[rt][j]), bl,
                                                                          acc[rt][tt], 0, 0, 0);
            }
        }
        if (c + 1 < nch) {
#pragma unroll
            for (int rt = 0; rt < GM_RT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) wc[rt][j] = wn[rt][j];
        }
    }

    // the lane holds rows 4q .. 4q+3 of each row tile for token 16 tt + c16
    if (a.S > 1) {
#pragma unroll
        for (int rt = 0; rt < GM_RT; ++rt) {
            const int n0 = gm_row(a, rb, wave, rt, 4 * q);
            if (n0 >= a.N) continue;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = t0 + tt * 16 + c16;
                *reinterpret_cast<float4 *>(a.part + ((int64_t)split * a.TP + t) * a.N + n0) =
                    make_float4(acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]);
            }
        }
        return;
    }
    if (a.epi == DM_EPI_SWIGLU) {
        const int half = a.N / 2;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int n0 = gm_row(a, rb, wave, rt, 4 * q);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = t0 + tt * 16 + c16;
                if (t >= a.T) continue;
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float g = acc[rt][tt][e], u = acc[rt + 2][tt][e];
                    o[e] = g / (1.0f + expf(-g)) * u;
                }
                *reinterpret_cast<float4 *>(a.y + (int64_t)t * half + n0) = make_float4(o[0], o[1], o[2], o[3]);
            }
        }
        return;
    }
#pragma unroll
    for (int rt = 0; rt < GM_RT; ++rt) {
        const int n0 = gm_row(a, rb, wave, rt, 4 * q);
        if (n0 >= a.N) continue;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int t = t0 + tt * 16 + c16;
            if (t >= a.T) continue;
            float4 *dst = reinterpret_cast<float4 *>(a.y + (int64_t)t * a.N + n0);
            float4 v = make_float4(acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]);
            if (a.epi == DM_EPI_ADD) {
                const float4 r = *dst;
                v.x += r.x;
                v.y += r.y;
                v.z += r.z;
                v.w += r.w;
            }
            *dst = v;
        }
    }
}

// y[t][n] (+)= the sum over splits in split order (SwiGLU: rows n and n + N/2)
__global__ __launch_bounds__(256) void gm_reduce_kernel(const float *part, int S, int TP, int N, int epi,
                                                        float *y)
{
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
    if (n >= n_out) return;
    float s = 0.f, u = 0.f;
    for (int sp = 0; sp < S; ++sp) {
        const float *p = part + ((int64_t)sp * TP + t) * N;
        s += p[n];
        if (epi == DM_EPI_SWIGLU) u += p[n + n_out];
    }
    float *dst = y + (int64_t)t * n_out + n;
    if (epi == DM_EPI_SWIGLU) *dst = s / (1.0f + expf(-s)) * u;
    else if (epi == DM_EPI_ADD) *dst += s;
    else *dst = s;
}

// tokens per block: 128 for long chunks (measured on the 512-token prompt of
// the 3.7B-shaped model: 23.1 ms against 24.2 with 64), less for short
// ones, whose padding would be wasted work
static int gm_bt(int T) { return T <= 32 ? 32 : T <= 64 ? 64 : 128; }
static int gm_tp(int T)
{
    const int bt = gm_bt(T);
    return (T + bt - 1) / bt * bt;
}
static int gm_rb(int N, int epi) { return epi == DM_EPI_SWIGLU ? N / GM_BM : (N + GM_BM - 1) / GM_BM; }

// Split-K count: one split when the row x token blocks already give a block
// per CU; else the most splits (a divisor of the chunk count, >= 2 chunks
// each) whose blocks still fit on the chip at once.
static int gm_splits(int N, int K, int T, int epi)
{
    const int bt = gm_bt(T);
    const int blk = gm_rb(N, epi) * (gm_tp(T) / bt);
    const int slots = 256 * (bt <= 64 ? 2 : 1);
    if (blk >= 256) return 1;
    const int nch = K / GM_BK;
    int S = 1;
    for (int s = 2; s <= nch / 2; ++s)
        if (nch % s == 0 && blk * s <= slots) S = s;
    return S;
}

bool gemm_mfma_ok(int N, int K, int epi)
{
    if (K % GM_BK || N < 16) return false;
    if (epi == DM_EPI_SWIGLU) return N % GM_BM == 0;
    return N % 4 == 0;
}

size_t gemm_mfma_ws_bytes(int N, int K, int T, int epi)
{
    if (!gemm_mfma_ok(N, K, epi) || T < 1 || T > GM_MAX_T) return 0;
    const int TP = gm_tp(T), S = gm_splits(N, K, T, epi);
    return 2 * k2_align256((size_t)TP * K * 2) + (S > 1 ? k2_align256((size_t)S * TP * N * 4) : 0);
}

int gemm_mfma(const uint16_t *W, const float *x, float *y, int N, int K, int T, int epi, void *ws,
              hipStream_t st)
{
    if (!gemm_mfma_ok(N, K, epi) || T < 1 || T > GM_MAX_T || !ws) return K2_EUNSUPPORTED;
    GemmArgs a{};
    const int BT = gm_bt(T), TP = gm_tp(T);
    const int S = gm_splits(N, K, T, epi);
    char *p = (char *)ws;
    uint16_t *xh = (uint16_t *)p;
    p += k2_align256((size_t)TP * K * 2);
    uint16_t *xl = (uint16_t *)p;
    p += k2_align256((size_t)TP * K * 2);
    a.W = W;
    a.xh = xh;
    a.xl = xl;
    a.part = S > 1 ? (float *)p : nullptr;
    a.y = y;
    a.N = N;
    a.K = K;
    a.T = T;
    a.TP = TP;
    a.S = S;
    a.KS = K / S;
    a.epi = epi;
    a.rb = gm_rb(N, epi);
    a.tb = TP / BT;
    const int nblk = a.rb * a.tb * S;
    a.xcd = nblk % 8 == 0;

    const int64_t n4 = (int64_t)TP * K / 4;
    int sb = (int)((n4 + 255) / 256);
    sb = sb < 2048 ? sb : 2048;
    hipLaunchKernelGGL(gm_split_kernel, dim3(sb), dim3(256), 0, st, x, xh, xl, T, TP, K);
    K2_CHECK_LAUNCH();
    const size_t lds = 2 * 2 * (size_t)BT * GM_ROWB;
    if (BT == 32) hipLaunchKernelGGL((gm_kernel<32>), dim3(nblk), dim3(256), lds, st, a);
    else if (BT == 64) hipLaunchKernelGGL((gm_kernel<64>), dim3(nblk), dim3(256), lds, st, a);
    else hipLaunchKernelGGL((gm_kernel<128>), dim3(nblk), dim3(256), lds, st, a);
    K2_CHECK_LAUNCH();
    if (S > 1) {
        const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
        hipLaunchKernelGGL(gm_reduce_kernel, dim3((n_out + 255) / 256, T), dim3(256), 0, st, a.part, S, TP, N,
                           epi, y);
        K2_CHECK_LAUNCH();
    }
    return K2_OK;
}

}  // namespace k2
