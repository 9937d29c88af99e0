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
//
// Quantized weights ([k2-burn] "Quantization": fp8 and int4 Q4S; [k3_run.c]
// header: MXFP4) are decoded in registers to bf16 values that are exact:
//   * fp8 E4M3: the code's value (3 mantissa bits); the row scale multiplies
//     the row's sum (the epilogue, or each split's partial);
//   * MXFP4: the E2M1 value times the block's 2^e (two significant bits);
//   * Q4S: the int4 code / 16; each 64-column block's products go to a
//     fresh accumulator that is added to the row's sum times 16 s[n][b].
// Which k a lane holds is free as long as A and B agree, so the quantized
// forms pick the k order that makes a lane's weight bytes contiguous (one
// or two 16- or 8-byte loads per row tile and chunk) and, for Q4S, keeps
// every MFMA inside one 64-column block; the LDS k-chunk read for B follows
// the same order.
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
    const void *W;             // [N][K] of the weight format (4-bit: [N][K/2] bytes)
    const void *Ws;            // fp8: float [N]; MXFP4: uint8 [N][K/32]; Q4S: float [N][K/64]
    const uint16_t *xh, *xl;   // [TP][K] bf16 planes (rows >= T zero)
    float *y;                  // [T][N] (SwiGLU: [T][N/2])
    uint16_t *yh, *yl;         // SwiGLU into bf16 hi / lo planes [T][N/2] instead of y (nullable)
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

// y, or its bf16 hi / lo planes, at element i
__device__ __forceinline__ void gm_out(const GemmArgs &a, int64_t i, float v)
{
    if (a.yh) {
        const uint16_t h = f32_to_bf16_rne(v);
        a.yh[i] = h;
        a.yl[i] = f32_to_bf16_rne(v - bf16_to_f32(h));
    } else {
        a.y[i] = v;
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

// two fp32 whose low 16 bits are zero (exact bf16 values) -> a bf16 pair
__device__ __forceinline__ uint32_t gm_pack(float lo, float hi)
{
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// bytes of weight storage per row per 128-column chunk; 16-byte registers
// per lane and row tile that hold a chunk's weights
template <int WDT> struct GmW;
template <> struct GmW<K2_BF16>    { static constexpr int CB = 256, NW = 4; };
template <> struct GmW<K2_FP8E4M3> { static constexpr int CB = 128, NW = 2; };
template <> struct GmW<K2_MXFP4>   { static constexpr int CB = 64,  NW = 1; };
template <> struct GmW<K2_Q4S>     { static constexpr int CB = 64,  NW = 1; };

// LDS k-chunk (8 columns) that lane quarter q multiplies in k-step j
template <int WDT>
__device__ __forceinline__ int gm_kchunk(int j, int q)
{
    if constexpr (WDT == K2_BF16) return 4 * j + q;                       // k = 32 j + 8 q
    else if constexpr (WDT == K2_Q4S) return 8 * (j >> 1) + 2 * q + (j & 1);   // k = 64 (j/2) + 16 q + 8 (j%2)
    else return 4 * q + j;                                                // k = 32 q + 8 j
}

// the lane's 8 weights of k-step j of one row tile, as exact bf16
template <int WDT>
__device__ __forceinline__ gm_bf16x8 gm_decode(const k2_u4 (&w)[GmW<WDT>::NW], int j, float sc)
{
    k2_u4 r;
    if constexpr (WDT == K2_BF16) {
        r = w[j];
    } else if constexpr (WDT == K2_FP8E4M3) {
        const k2_u4 u = w[j >> 1];
        const uint32_t d0 = (j & 1) ? u.z : u.x, d1 = (j & 1) ? u.w : u.y;
        const k2_f2 a = fp8x2_lo(d0), b = fp8x2_hi(d0), c = fp8x2_lo(d1), d = fp8x2_hi(d1);
        r = k2_u4{gm_pack(a.x, a.y), gm_pack(b.x, b.y), gm_pack(c.x, c.y), gm_pack(d.x, d.y)};
    } else if constexpr (WDT == K2_MXFP4) {
        const uint32_t d = w[0][j];
        const k2_f2 a = fp4x2<0>(d), b = fp4x2<1>(d), c = fp4x2<2>(d), e = fp4x2<3>(d);
        r = k2_u4{gm_pack(a.x * sc, a.y * sc), gm_pack(b.x * sc, b.y * sc), gm_pack(c.x * sc, c.y * sc),
                  gm_pack(e.x * sc, e.y * sc)};
    } else {
        const uint32_t d = w[0][j];
        r = k2_u4{gm_pack(q4s_off(d), q4s_off(d >> 4)), gm_pack(q4s_off(d >> 8), q4s_off(d >> 12)),
                  gm_pack(q4s_off(d >> 16), q4s_off(d >> 20)), gm_pack(q4s_off(d >> 24), q4s_off(d >> 28))};
    }
    return __builtin_bit_cast(gm_bf16x8, r);
}

template <int BT, int WDT>
__global__ __launch_bounds__(256, BT <= 64 ? 2 : 1) void gm_kernel(const GemmArgs a)
{
    constexpr int NT = BT / 16;                           // token tiles
    constexpr int PLANE = BT * GM_ROWB;                   // bytes of one plane's chunk tile
    constexpr int STAGE = 2 * PLANE;                      // hi + lo
    constexpr int NDMA = PLANE / 1024 / 4;                // 1 KiB wave copies per wave, plane and chunk
    constexpr int CB = GmW<WDT>::CB, NW = GmW<WDT>::NW;
    constexpr bool Q4 = WDT == K2_Q4S;
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
    const int64_t rowb = (int64_t)a.K / GM_BK * CB;       // storage bytes of one row

    // this wave's row tiles (A rows: lane row c16); rows past N read row N-1
    // and are never stored.  Byte offset of the lane's first load in chunk 0:
    // bf16 k = 8q (then +32 per k-step), fp8 k = 32q, MXFP4 k = 32q, Q4S
    // k = 16q (then +64 for the second block)
    const char *wrow[GM_RT];
    const uint32_t *erow[GM_RT];                          // MXFP4: the row's scale bytes of chunk 0
    constexpr int QOFF = WDT == K2_BF16 ? 16 : WDT == K2_FP8E4M3 ? 32 : WDT == K2_MXFP4 ? 16 : 8;
#pragma unroll
    for (int rt = 0; rt < GM_RT; ++rt) {
        int r = gm_row(a, rb, wave, rt, c16);
        r = r < a.N ? r : a.N - 1;
        wrow[rt] = (const char *)a.W + r * rowb + (int64_t)kbeg / GM_BK * CB + q * QOFF;
        if constexpr (WDT == K2_MXFP4)
            erow[rt] = (const uint32_t *)((const uint8_t *)a.Ws + (int64_t)r * (a.K / 32) + kbeg / 32);
    }
    // Q4S: the lane's row's block scales (the product is taken transposed,
    // so a lane's D values all belong to its own weight row c16)
    const float *srow[GM_RT];
    if constexpr (Q4) {
#pragma unroll
        for (int rt = 0; rt < GM_RT; ++rt) {
            int r = gm_row(a, rb, wave, rt, c16);
            r = r < a.N ? r : a.N - 1;
            srow[rt] = (const float *)a.Ws + (int64_t)r * (a.K / 64) + kbeg / 64;
        }
    }
    // (scales stay raw until used: converting them here would wait for the
    // loads just issued)
    auto load_w = [&](int c, k2_u4 (&w)[GM_RT][NW], uint32_t (&e)[GM_RT], k2_f2 (&s)[GM_RT]) {
#pragma unroll
        for (int rt = 0; rt < GM_RT; ++rt) {
            const char *p = wrow[rt] + (int64_t)c * CB;
            if constexpr (WDT == K2_BF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[rt][j] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(p + 64 * j));
            } else if constexpr (WDT == K2_FP8E4M3) {
                w[rt][0] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(p));
                w[rt][1] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(p + 16));
            } else if constexpr (WDT == K2_MXFP4) {
                w[rt][0] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(p));
                e[rt] = erow[rt][c];
            } else {
                const uint64_t lo = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(p));
                const uint64_t hi = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(p + 32));
                w[rt][0] = k2_u4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
                s[rt] = *reinterpret_cast<const k2_f2 *>(srow[rt] + 2 * c);
            }
        }
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

    k2_u4 wc[GM_RT][NW], wn[GM_RT][NW];
    uint32_t ec[GM_RT], en[GM_RT];
    k2_f2 sc[GM_RT], sn[GM_RT];
    load_w(0, wc, ec, sc);
    dma_x(0);
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        __builtin_amdgcn_s_waitcnt(0);                    // this wave's copies of chunk c and its weights are in
        __syncthreads();                                  // every wave's; nobody still reads buffer (c + 1) & 1
        if (c + 1 < nch) {
            dma_x(c + 1);
            load_w(c + 1, wn, en, sn);
        }
        const char *st = lds + (c & 1) * STAGE;
        if constexpr (!Q4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gm_bf16x8 A[GM_RT];
#pragma unroll
                for (int rt = 0; rt < GM_RT; ++rt)
                    A[rt] = gm_decode<WDT>(wc[rt], j, WDT == K2_MXFP4 ? e8m0_to_f32((ec[rt] >> (8 * q)) & 0xFFu) : 0.f);
                const int kc = gm_kchunk<WDT>(j, q);          // this lane's k-chunk in k-step j
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
                        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rt], bh, acc[rt][tt], 0, 0, 0);
#pragma unroll
                    for (int rt = 0; rt < GM_RT; ++rt)
                        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rt], bl, acc[rt][tt], 0, 0, 0);
                }
            }
        } else {
            // two 64-column blocks per chunk: each block's four MFMAs (two
            // k-steps, hi and lo) into a fresh accumulator, then scaled in.
            // Operands swapped (D = X W^T): lane l holds tokens 4 (l / 16) +
            // [0, 4) of weight row l % 16, so one scale per lane and block
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                gm_bf16x8 A0[GM_RT], A1[GM_RT];
#pragma unroll
                for (int rt = 0; rt < GM_RT; ++rt) {
                    A0[rt] = gm_decode<WDT>(wc[rt], 2 * h, 0.f);
                    A1[rt] = gm_decode<WDT>(wc[rt], 2 * h + 1, 0.f);
                }
                const int kc0 = gm_kchunk<WDT>(2 * h, q), kc1 = gm_kchunk<WDT>(2 * h + 1, q);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int t = tt * 16 + c16;
                    const int o0 = t * GM_ROWB + ((kc0 - t) & 15) * 16, o1 = t * GM_ROWB + ((kc1 - t) & 15) * 16;
                    const gm_bf16x8 bh0 = *reinterpret_cast<const gm_bf16x8 *>(st + o0);
                    const gm_bf16x8 bl0 = *reinterpret_cast<const gm_bf16x8 *>(st + PLANE + o0);
                    const gm_bf16x8 bh1 = *reinterpret_cast<const gm_bf16x8 *>(st + o1);
                    const gm_bf16x8 bl1 = *reinterpret_cast<const gm_bf16x8 *>(st + PLANE + o1);
                    gm_f32x4 tmp[GM_RT];
#pragma unroll
                    for (int rt = 0; rt < GM_RT; ++rt)
                        tmp[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh0, A0[rt], gm_f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                         0, 0);
#pragma unroll
                    for (int rt = 0; rt < GM_RT; ++rt)
                        tmp[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl0, A0[rt], tmp[rt], 0, 0, 0);
#pragma unroll
                    for (int rt = 0; rt < GM_RT; ++rt)
                        tmp[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh1, A1[rt], tmp[rt], 0, 0, 0);
#pragma unroll
                    for (int rt = 0; rt < GM_RT; ++rt)
                        tmp[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl1, A1[rt], tmp[rt], 0, 0, 0);
#pragma unroll
                    for (int rt = 0; rt < GM_RT; ++rt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[rt][tt][e] += tmp[rt][e] * (16.0f * sc[rt][h]);
                    // one token tile at a time: the scheduler would otherwise
                    // start the next tiles' reads and chains early, past the
                    // register budget
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (c + 1 < nch) {
#pragma unroll
            for (int rt = 0; rt < GM_RT; ++rt) {
#pragma unroll
                for (int j = 0; j < NW; ++j) wc[rt][j] = wn[rt][j];
                ec[rt] = en[rt];
                sc[rt] = sn[rt];
            }
        }
    }

    // fp8: the row scales of the lane's D rows 4q .. 4q+3
    if constexpr (WDT == K2_FP8E4M3) {
#pragma unroll
        for (int rt = 0; rt < GM_RT; ++rt) {
            const int n0 = gm_row(a, rb, wave, rt, 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + e < a.N ? n0 + e : a.N - 1;
                const float rs = ((const float *)a.Ws)[n];
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) acc[rt][tt][e] *= rs;
            }
        }
    }

    if constexpr (Q4) {
        // the lane holds row c16 of each row tile for tokens 16 tt + 4q + [0, 4)
        if (a.S > 1) {
#pragma unroll
            for (int rt = 0; rt < GM_RT; ++rt) {
                const int n = gm_row(a, rb, wave, rt, c16);
                if (n >= a.N) continue;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = t0 + tt * 16 + 4 * q + e;
                        a.part[((int64_t)split * a.TP + t) * a.N + n] = acc[rt][tt][e];
                    }
            }
            return;
        }
        if (a.epi == DM_EPI_SWIGLU) {
            const int half = a.N / 2;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int n = gm_row(a, rb, wave, rt, c16);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = t0 + tt * 16 + 4 * q + e;
                        if (t >= a.T) continue;
                        const float g = acc[rt][tt][e], u = acc[rt + 2][tt][e];
                        gm_out(a, (int64_t)t * half + n, g / (1.0f + expf(-g)) * u);
                    }
            }
            return;
        }
#pragma unroll
        for (int rt = 0; rt < GM_RT; ++rt) {
            const int n = gm_row(a, rb, wave, rt, c16);
            if (n >= a.N) continue;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = t0 + tt * 16 + 4 * q + e;
                    if (t >= a.T) continue;
                    float *dst = a.y + (int64_t)t * a.N + n;
                    *dst = a.epi == DM_EPI_ADD ? *dst + acc[rt][tt][e] : acc[rt][tt][e];
                }
        }
        return;
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
                const int64_t i0 = (int64_t)t * half + n0;
                if (a.yh) {
                    uint16_t h[4], l[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[e] = f32_to_bf16_rne(o[e]);
                        l[e] = f32_to_bf16_rne(o[e] - bf16_to_f32(h[e]));
                    }
                    *reinterpret_cast<uint2 *>(a.yh + i0) =
                        make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                    *reinterpret_cast<uint2 *>(a.yl + i0) =
                        make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
                } else {
                    *reinterpret_cast<float4 *>(a.y + i0) = make_float4(o[0], o[1], o[2], o[3]);
                }
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
                                                        float *y, uint16_t *yh, uint16_t *yl)
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
    const int64_t i = (int64_t)t * n_out + n;
    if (epi == DM_EPI_SWIGLU) {
        const float v = s / (1.0f + expf(-s)) * u;
        if (yh) {
            const uint16_t h = f32_to_bf16_rne(v);
            yh[i] = h;
            yl[i] = f32_to_bf16_rne(v - bf16_to_f32(h));
        } else {
            y[i] = v;
        }
    } else if (epi == DM_EPI_ADD) {
        y[i] += s;
    } else {
        y[i] = s;
    }
}

// tokens per block: 128 for long chunks (measured on the 512-token prompt of
// the 3.7B-shaped model: 23.1 ms against 24.2 with 64), less for short
// ones, whose padding would be wasted work.  Q4S: 32 (its fresh per-block
// accumulators and the scaled sums need registers that larger token blocks
// would spill)
static int gm_bt(int T, int wdt)
{
    if (wdt == K2_Q4S) return 32;
    return T <= 32 ? 32 : T <= 64 ? 64 : 128;
}
static int gm_tp(int T, int wdt)
{
    const int bt = gm_bt(T, wdt);
    return (T + bt - 1) / bt * bt;
}
static int gm_rb(int N, int epi) { return epi == DM_EPI_SWIGLU ? N / GM_BM : (N + GM_BM - 1) / GM_BM; }

// Split-K count: one split when the row x token blocks already give a block
// per CU; else the most splits (a divisor of the chunk count, >= 2 chunks
// each) whose blocks still fit on the chip at once.
static int gm_splits(int N, int K, int T, int epi, int wdt)
{
    const int bt = gm_bt(T, wdt);
    const int blk = gm_rb(N, epi) * (gm_tp(T, wdt) / bt);
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

size_t gemm_mfma_ws_bytes(int wdt, int N, int K, int T, int epi)
{
    if (!gemm_mfma_ok(N, K, epi) || T < 1 || T > GM_MAX_T) return 0;
    const int TP = gm_tp(T, wdt), S = gm_splits(N, K, T, epi, wdt);
    return 2 * k2_align256((size_t)TP * K * 2) + (S > 1 ? k2_align256((size_t)S * TP * N * 4) : 0);
}

template <int WDT>
static void gm_launch(int BT, int nblk, size_t lds, hipStream_t st, const GemmArgs &a)
{
    if constexpr (WDT == K2_Q4S) {
        hipLaunchKernelGGL((gm_kernel<32, WDT>), dim3(nblk), dim3(256), lds, st, a);
    } else {
        if (BT == 32) hipLaunchKernelGGL((gm_kernel<32, WDT>), dim3(nblk), dim3(256), lds, st, a);
        else if (BT == 64) hipLaunchKernelGGL((gm_kernel<64, WDT>), dim3(nblk), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((gm_kernel<128, WDT>), dim3(nblk), dim3(256), lds, st, a);
    }
}

// The product from activation planes xh / xl [>= TP rows][K] (rows past T
// may hold anything: a token's outputs depend on its own row only, and rows
// past T are neither stored nor summed).  ws: gemm_mfma_ws_bytes (its
// plane part unused here).
static int gm_core(int wdt, const void *W, const void *Ws, const uint16_t *xh, const uint16_t *xl, float *y,
                   uint16_t *yh, uint16_t *yl, int N, int K, int T, int epi, void *ws, hipStream_t st)
{
    GemmArgs a{};
    const int BT = gm_bt(T, wdt), TP = gm_tp(T, wdt);
    const int S = gm_splits(N, K, T, epi, wdt);
    char *p = (char *)ws + 2 * k2_align256((size_t)TP * K * 2);
    a.W = W;
    a.Ws = Ws;
    a.xh = xh;
    a.xl = xl;
    a.part = S > 1 ? (float *)p : nullptr;
    a.y = y;
    a.yh = yh;
    a.yl = yl;
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
    const size_t lds = 2 * 2 * (size_t)BT * GM_ROWB;
    switch (wdt) {
    case K2_BF16: gm_launch<K2_BF16>(BT, nblk, lds, st, a); break;
    case K2_FP8E4M3: gm_launch<K2_FP8E4M3>(BT, nblk, lds, st, a); break;
    case K2_MXFP4: gm_launch<K2_MXFP4>(BT, nblk, lds, st, a); break;
    default: gm_launch<K2_Q4S>(BT, nblk, lds, st, a); break;
    }
    K2_CHECK_LAUNCH();
    if (S > 1) {
        const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
        hipLaunchKernelGGL(gm_reduce_kernel, dim3((n_out + 255) / 256, T), dim3(256), 0, st, a.part, S, TP, N,
                           epi, y, yh, yl);
        K2_CHECK_LAUNCH();
    }
    return K2_OK;
}

static int gm_check(int wdt, const void *Ws, int N, int K, int T, int epi, const void *ws)
{
    if (!gemm_mfma_ok(N, K, epi) || T < 1 || T > GM_MAX_T || !ws) return K2_EUNSUPPORTED;
    if (wdt != K2_BF16 && wdt != K2_FP8E4M3 && wdt != K2_MXFP4 && wdt != K2_Q4S) return K2_EUNSUPPORTED;
    if (wdt != K2_BF16 && !Ws) return K2_EINVAL;
    return K2_OK;
}

int gemm_mfma(int wdt, const void *W, const void *Ws, const float *x, float *y, int N, int K, int T, int epi,
              void *ws, hipStream_t st)
{
    int rc = gm_check(wdt, Ws, N, K, T, epi, ws);
    if (rc) return rc;
    const int TP = gm_tp(T, wdt);
    uint16_t *xh = (uint16_t *)ws;
    uint16_t *xl = (uint16_t *)((char *)ws + k2_align256((size_t)TP * K * 2));
    const int64_t n4 = (int64_t)TP * K / 4;
    int sb = (int)((n4 + 255) / 256);
    sb = sb < 2048 ? sb : 2048;
    hipLaunchKernelGGL(gm_split_kernel, dim3(sb), dim3(256), 0, st, x, xh, xl, T, TP, K);
    K2_CHECK_LAUNCH();
    return gm_core(wdt, W, Ws, xh, xl, y, nullptr, nullptr, N, K, T, epi, ws, st);
}

int gemm_mfma_planes(int wdt, const void *W, const void *Ws, const uint16_t *xh, const uint16_t *xl, float *y,
                     uint16_t *yh, uint16_t *yl, int N, int K, int T, int epi, void *ws, hipStream_t st)
{
    int rc = gm_check(wdt, Ws, N, K, T, epi, ws);
    if (rc) return rc;
    if (!xh || !xl || ((yh || yl) && (epi != DM_EPI_SWIGLU || !yh || !yl))) return K2_EINVAL;
    return gm_core(wdt, W, Ws, xh, xl, y, yh, yl, N, K, T, epi, ws, st);
}

int gemm_mfma_rows(int T, int wdt) { return gm_tp(T, wdt); }

}  // namespace k2
