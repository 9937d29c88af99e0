// dense_mfma.hip -- a bf16 weight matrix times a few fp32 activation rows
// (2 to 32 tokens at a time) on the matrix cores.
//
// The latent-MoE layer ([k3_run.c] forward(): router, W_dn, W_up and the
// shared experts) multiplies every dense matrix by T token rows.  With T rows
// a weight byte feeds 2T flops; past a few tokens that outgrows fp32 vector
// arithmetic, so here the product runs on v_mfma_f32_16x16x32_bf16:
//   * each activation is split into bf16 hi + bf16 lo (x - hi rounded again),
//     two MFMAs per weight tile, fp32 accumulation: the weights are exact in
//     bf16 and the split keeps ~16 bits of every activation;
//   * a block of 4 waves owns 256, 128 or 64 rows and one k-range (split-K); it stages
//     its slice of the activations once in LDS as the two bf16 planes, each
//     wave streams its 4, 2 or 1 row tiles of 16 rows from HBM, one 128-column chunk
//     ahead of the MFMAs;
//   * per-split partials [split][token][row] are summed in split order by a
//     second kernel, which also applies the epilogue (plain, add into y, or
//     SwiGLU of row pairs i, i + N/2) -- or, given arrival counters, by the
//     last block to finish of each row block (of each gate / up row-block
//     pair for SwiGLU): every block stores its partials at device scope and
//     counts itself, and the last one sums the group's partials in split
//     order (the same order, so the same result) and applies the epilogue.
//     That saves the second launch, whose gap and first-byte latency are
//     most of its cost at these sizes.
// MFMA operand layout (16x16x32 bf16): lane l holds A row l % 16 and B column
// l % 16, elements k = 8 (l / 16) + [0, 8); D holds column l % 16, rows
// 4 (l / 16) + [0, 4).
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

typedef short dm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float dm_f32x4 __attribute__((ext_vector_type(4)));

constexpr int DM_WAVES = 4;                       // waves per block
constexpr int DM_MIN_ROWS = 16 * DM_WAVES;        // rows per block with one 16-row tile per wave
constexpr int DM_KC = 128;                        // columns per chunk (4 MFMA k-steps)
constexpr int DM_MAX_T = 32;                      // tokens per launch
constexpr int DM_FUSE_MAX = 128;                  // tokens x splits summed in-kernel at most

struct DenseArgs {
    const uint16_t *W;       // [N][K] bf16
    const float *x;          // [T][K] fp32
    float *part;             // [splits][TP][N]
    int N, K, T, KS;
    // in-kernel reduction (cnt non-null): arrival counters [groups], zero
    // between launches; the epilogue and its output y [T][N or N/2]
    unsigned *cnt;
    float *y;
    int epi;
};

__host__ __device__ constexpr int dm_lds_bytes(int tp, int ks) { return 2 * tp * (ks + 8) * 2; }

template <int NTT, int KS, int RT>
__global__ __launch_bounds__(256) void dense_mfma_kernel(const DenseArgs a)
{
    constexpr int ROWS = RT * 16 * DM_WAVES;      // rows per block
    constexpr int TP = 16 * NTT;
    constexpr int RS = KS + 8;                    // LDS row stride (bf16): 16 B of pad per row
    constexpr int NCH = KS / DM_KC;               // chunks per split
    constexpr int NG = TP * KS / 4 / 256;         // activation float4s per thread
    extern __shared__ float4 lds4[];
    uint16_t *xh = reinterpret_cast<uint16_t *>(lds4);
    uint16_t *xl = xh + TP * RS;
    const int split = blockIdx.y, k0 = split * KS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, c16 = lane & 15;

    // rows of this wave's tiles (tiles past N read the last tile again and
    // are never stored)
    int64_t rowoff[RT];
    bool rok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r0 = blockIdx.x * ROWS + (wave * RT + rt) * 16;
        rok[rt] = r0 < a.N;
        const int row = (rok[rt] ? r0 : a.N - 16) + c16;
        rowoff[rt] = (int64_t)row * a.K + k0 + q * 8;
    }
    const dm_bf16x8 *Wv = reinterpret_cast<const dm_bf16x8 *>(a.W);
    // chunk c of tile rt, k-step j: the 16 B at element rowoff + c*128 + 32j
    // (the 4 lanes of a row read 64 contiguous bytes per instruction)
    auto load_chunk = [&](int c, dm_bf16x8 (&w)[RT][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[rt][j] = __builtin_nontemporal_load(Wv + (rowoff[rt] + c * DM_KC + 32 * j) / 8);
    };
    dm_bf16x8 wc[RT][4];
    load_chunk(0, wc);                            // weights first: their latency covers the staging

    // stage the activation slice as bf16 hi / lo planes (tokens >= T are 0):
    // every load is issued before any is converted
    float4 xv[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int i = g * 256 + tid, t = i / (KS / 4), k = (i % (KS / 4)) * 4;
        xv[g] = t < a.T ? *reinterpret_cast<const float4 *>(a.x + (int64_t)t * a.K + k0 + k)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int i = g * 256 + tid, t = i / (KS / 4), k = (i % (KS / 4)) * 4;
        const float f[4] = {xv[g].x, xv[g].y, xv[g].z, xv[g].w};
        uint16_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = f32_to_bf16_rne(f[e]);
            l[e] = f32_to_bf16_rne(f[e] - bf16_to_f32(h[e]));
        }
        uint2 hv, lv;
        hv.x = h[0] | ((uint32_t)h[1] << 16); hv.y = h[2] | ((uint32_t)h[3] << 16);
        lv.x = l[0] | ((uint32_t)l[1] << 16); lv.y = l[2] | ((uint32_t)l[3] << 16);
        *reinterpret_cast<uint2 *>(xh + t * RS + k) = hv;
        *reinterpret_cast<uint2 *>(xl + t * RS + k) = lv;
    }
    __syncthreads();

    dm_f32x4 acc[RT][NTT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = dm_f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c, const dm_bf16x8 (&w)[RT][4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = c * DM_KC + 32 * j + q * 8;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int t = tt * 16 + c16;
                const dm_bf16x8 bh = *reinterpret_cast<const dm_bf16x8 *>(xh + t * RS + kk);
                const dm_bf16x8 bl = *reinterpret_cast<const dm_bf16x8 *>(xl + t * RS + kk);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[rt][j], bh, acc[rt][tt], 0, 0, 0);
                    acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[rt][j], bl, acc[rt][tt], 0, 0, 0);
                }
            }
        }
    };
    // one chunk ahead of the MFMAs; the last chunk without a next one
#pragma unroll 1
    for (int c = 0; c + 1 < NCH; ++c) {
        dm_bf16x8 wn[RT][4];
        load_chunk(c + 1, wn);
        compute(c, wc);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) wc[rt][j] = wn[rt][j];
    }
    compute(NCH - 1, wc);

    // partials: the lane holds rows 4q..4q+3 of each tile for token c16 + 16 tt
    // (device scope when another block sums them)
    const bool fuse = a.cnt != nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (!rok[rt]) continue;
        const int r0 = blockIdx.x * ROWS + (wave * RT + rt) * 16 + 4 * q;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = tt * 16 + c16;
            if (t >= a.T) continue;
            const int64_t o = ((int64_t)split * TP + t) * a.N + r0;
            const float4 v = make_float4(acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]);
            if (fuse) coh_store4(a.part, (int)o, v);
            else *reinterpret_cast<float4 *>(a.part + o) = v;
        }
    }
    if (!fuse) return;

    // arrival: row block b alone, or SwiGLU gate block b with up block
    // b + rb / 2 (both counted on counter b)
    __shared__ int last;
    const int rb = gridDim.x, splits = gridDim.y;
    const bool pair = a.epi == DM_EPI_SWIGLU;
    const int grp = pair ? blockIdx.x % (rb / 2) : blockIdx.x;
    const unsigned arrivals = (unsigned)(pair ? 2 * splits : splits);
    __builtin_amdgcn_s_waitcnt(0);                // this thread's partial stores completed
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == arrivals - 1;
        if (last) __hip_atomic_store(a.cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;

    // the group's outputs, each summed over the splits in split order: a
    // thread owns 4 consecutive outputs (gate rows for SwiGLU) of every
    // TSTEP-th token and loads 8 splits' partials before adding them
    constexpr int QUADS = ROWS / 4, TSTEP = 256 / QUADS;
    const int n_out = pair ? a.N / 2 : a.N;
    const int n = grp * ROWS + (tid % QUADS) * 4;
    if (n >= n_out) return;
    constexpr int B8 = 8;
    for (int t = tid / QUADS; t < a.T; t += TSTEP) {
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f), up = sum;
        for (int s0 = 0; s0 < splits; s0 += B8) {
            float4 v[B8], u[B8];
#pragma unroll
            for (int i = 0; i < B8; ++i) {
                if (s0 + i >= splits) break;
                const int o = (int)(((int64_t)(s0 + i) * TP + t) * a.N + n);
                v[i] = coh_load4(a.part, o);
                if (pair) u[i] = coh_load4(a.part, o + n_out);
            }
#pragma unroll
            for (int i = 0; i < B8; ++i) {
                if (s0 + i >= splits) break;
                sum.x += v[i].x; sum.y += v[i].y; sum.z += v[i].z; sum.w += v[i].w;
                if (pair) { up.x += u[i].x; up.y += u[i].y; up.z += u[i].z; up.w += u[i].w; }
            }
        }
        float4 *dst = reinterpret_cast<float4 *>(a.y + (int64_t)t * n_out + n);
        if (pair) {
            *dst = make_float4(sum.x / (1.0f + expf(-sum.x)) * up.x, sum.y / (1.0f + expf(-sum.y)) * up.y,
                               sum.z / (1.0f + expf(-sum.z)) * up.z, sum.w / (1.0f + expf(-sum.w)) * up.w);
        } else if (a.epi == DM_EPI_ADD) {
            const float4 r = *dst;
            *dst = make_float4(r.x + sum.x, r.y + sum.y, r.z + sum.z, r.w + sum.w);
        } else {
            *dst = sum;
        }
    }
}

// y[t][n] (+)= sum over splits in split order; SwiGLU: n < N/2 pairs rows n
// (gate) and n + N/2 (up) and y has N/2 columns.
__global__ __launch_bounds__(256) void dense_reduce_kernel(const float *part, int splits, int TP, int N,
                                                           int epi, float *y)
{
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
    if (n >= n_out) return;
    float s = 0.f, u = 0.f;
    for (int sp = 0; sp < splits; ++sp) {
        const float *p = part + ((int64_t)sp * TP + t) * N;
        s += p[n];
        if (epi == DM_EPI_SWIGLU) u += p[n + n_out];
    }
    float *dst = y + (int64_t)t * n_out + n;
    if (epi == DM_EPI_SWIGLU) *dst = s / (1.0f + expf(-s)) * u;
    else if (epi == DM_EPI_ADD) *dst += s;
    else *dst = s;
}

// Tile shape: 16-row tiles per wave (RT: 256, 128 or 64 rows per block) and
// columns per split (KS), the first of (4, 1024), (2, 1024), (1, 1024) (up
// to 16 tokens: with 32 their activation slice fills the LDS of a compute
// unit, and measured slower), (4, 512), (2, 512), (1, 512), (1, 256),
// (1, 128) that divides K and gives at least 256 blocks (else the last): the
// longest splits first (their chunks stream one ahead of the
// matrix cores, and fewer splits leave fewer partials), then the largest row
// blocks (an activation fragment read from LDS feeds RT row tiles).
struct DmTile { int rt, ks; };
static DmTile dm_tile(int N, int K, int T)
{
    static const DmTile cand[] = {{4, 1024}, {2, 1024}, {1, 1024}, {4, 512}, {2, 512},
                                  {1, 512},  {1, 256},  {1, 128}};
    const int tp = (T < DM_MAX_T ? T : DM_MAX_T) <= 16 ? 16 : 32;
    for (const DmTile &c : cand) {
        if (c.ks == 1024 && tp > 16) continue;
        const int64_t rb = (N + c.rt * DM_MIN_ROWS - 1) / (c.rt * DM_MIN_ROWS);
        if (K % c.ks == 0 && rb * (K / c.ks) >= 256) return c;
    }
    return {1, DM_KC};
}

bool dense_mfma_ok(int N, int K) { return N >= 16 && N % 16 == 0 && K % DM_KC == 0; }

size_t dense_mfma_ws_bytes(int N, int K, int T)
{
    if (!dense_mfma_ok(N, K) || T < 2) return 0;
    const int tp = (T < DM_MAX_T ? T : DM_MAX_T) <= 16 ? 16 : 32;
    return (size_t)(K / dm_tile(N, K, T).ks) * tp * N * 4;
}

int dense_mfma_cnt_words(int N) { return (N + DM_MIN_ROWS - 1) / DM_MIN_ROWS; }

template <int NTT, int KS>
static void dm_go(int rt, dim3 grid, size_t lds, hipStream_t st, const DenseArgs &a)
{
    if (rt == 4) hipLaunchKernelGGL((dense_mfma_kernel<NTT, KS, 4>), grid, dim3(256), lds, st, a);
    else if (rt == 2) hipLaunchKernelGGL((dense_mfma_kernel<NTT, KS, 2>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((dense_mfma_kernel<NTT, KS, 1>), grid, dim3(256), lds, st, a);
}

// y = W x for T token rows (T >= 2), through per-split partials in `part`
// (dense_mfma_ws_bytes); groups of up to 32 tokens run one after another.
// cnt (nullable, dense_mfma_cnt_words(N) zeroed words, left zero): sum the
// partials in the product's last blocks instead of a second launch (SwiGLU
// only when N / 2 is a multiple of the row block).
int dense_mfma(const uint16_t *W, const float *x, float *y, int N, int K, int T, int epi, float *part,
               hipStream_t st, unsigned *cnt)
{
    if (!dense_mfma_ok(N, K) || T < 2) return K2_EUNSUPPORTED;
    const DmTile tile = dm_tile(N, K, T);
    const int KS = tile.ks, splits = K / KS, rows = tile.rt * DM_MIN_ROWS;
    const int n_out = epi == DM_EPI_SWIGLU ? N / 2 : N;
    if (epi == DM_EPI_SWIGLU && (N / 2) % rows) cnt = nullptr;
    // the last block of a group reads T x splits partial rows: past ~128 of
    // them that tail costs more than the second launch (3.7B shape,
    // verification rounds with every product fused: T = 2 3.90 against 4.23
    // ms, T = 8 4.85 against 4.84, T = 16 5.85 against 5.12)
    if ((int64_t)(T < DM_MAX_T ? T : DM_MAX_T) * splits > DM_FUSE_MAX) cnt = nullptr;
    for (int t0 = 0; t0 < T; t0 += DM_MAX_T) {
        const int tg = T - t0 < DM_MAX_T ? T - t0 : DM_MAX_T;
        DenseArgs a{W, x + (int64_t)t0 * K, part, N, K, tg, KS, cnt, y + (int64_t)t0 * n_out, epi};
        const dim3 grid((N + rows - 1) / rows, splits);
        const int tp = tg <= 16 ? 16 : 32;
        const size_t lds = dm_lds_bytes(tp, KS);
        if (tp == 16) {
            if (KS == 1024) dm_go<1, 1024>(tile.rt, grid, lds, st, a);
            else if (KS == 512) dm_go<1, 512>(tile.rt, grid, lds, st, a);
            else if (KS == 256) dm_go<1, 256>(tile.rt, grid, lds, st, a);
            else dm_go<1, 128>(tile.rt, grid, lds, st, a);
        } else {
            if (KS == 1024) dm_go<2, 1024>(tile.rt, grid, lds, st, a);
            else if (KS == 512) dm_go<2, 512>(tile.rt, grid, lds, st, a);
            else if (KS == 256) dm_go<2, 256>(tile.rt, grid, lds, st, a);
            else dm_go<2, 128>(tile.rt, grid, lds, st, a);
        }
        K2_CHECK_LAUNCH();
        if (cnt) continue;
        hipLaunchKernelGGL(dense_reduce_kernel, dim3((n_out + 255) / 256, tg), dim3(256), 0, st, part,
                           splits, tp, N, epi, y + (int64_t)t0 * n_out);
        K2_CHECK_LAUNCH();
    }
    return K2_OK;
}

}  // namespace k2
