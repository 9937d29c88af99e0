// gemv_impl.h -- the templated GEMV kernel and its tile dispatch; included
// once per weight format by gemv_<format>.hip (one translation unit each,
// so the instantiations compile in parallel).
#pragma once
#include "k2_dev.h"
#include "k2_internal.h"

namespace k2 {

template <int WDT> struct WT;
template <> struct WT<K2_F32>     { static constexpr int EPC = 4;  };
template <> struct WT<K2_BF16>    { static constexpr int EPC = 8;  };
template <> struct WT<K2_FP8E4M3> { static constexpr int EPC = 16; };
template <> struct WT<K2_MXFP4>   { static constexpr int EPC = 32; };

// dot of one 16-byte weight chunk with EPC consecutive activations in LDS
template <int WDT>
__device__ __forceinline__ float chunk_dot(const k2_u4 w, const float *__restrict__ x)
{
    float s0 = 0.f, s1 = 0.f;
    if constexpr (WDT == K2_F32) {
        const float4 xv = *reinterpret_cast<const float4 *>(x);
        s0 = __uint_as_float(w.x) * xv.x + __uint_as_float(w.y) * xv.y;
        s1 = __uint_as_float(w.z) * xv.z + __uint_as_float(w.w) * xv.w;
    } else if constexpr (WDT == K2_BF16) {
        const float4 a = *reinterpret_cast<const float4 *>(x);
        const float4 b = *reinterpret_cast<const float4 *>(x + 4);
        s0 = bf16_lo(w.x) * a.x + bf16_hi(w.x) * a.y;
        s1 = bf16_lo(w.y) * a.z + bf16_hi(w.y) * a.w;
        s0 += bf16_lo(w.z) * b.x + bf16_hi(w.z) * b.y;
        s1 += bf16_lo(w.w) * b.z + bf16_hi(w.w) * b.w;
    } else if constexpr (WDT == K2_FP8E4M3) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 xv = *reinterpret_cast<const float4 *>(x + 4 * i);
            const k2_f2 lo = fp8x2_lo(ws[i]);
            const k2_f2 hi = fp8x2_hi(ws[i]);
            s0 += lo.x * xv.x + lo.y * xv.y;
            s1 += hi.x * xv.z + hi.y * xv.w;
        }
    } else {  // MXFP4: 32 E2M1 values, low nibble first
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 xa = *reinterpret_cast<const float4 *>(x + 8 * i);
            const float4 xb = *reinterpret_cast<const float4 *>(x + 8 * i + 4);
            const k2_f2 v0 = fp4x2<0>(ws[i]);
            const k2_f2 v1 = fp4x2<1>(ws[i]);
            const k2_f2 v2 = fp4x2<2>(ws[i]);
            const k2_f2 v3 = fp4x2<3>(ws[i]);
            s0 += v0.x * xa.x + v0.y * xa.y;
            s1 += v1.x * xa.z + v1.y * xa.w;
            s0 += v2.x * xb.x + v2.y * xb.y;
            s1 += v3.x * xb.z + v3.y * xb.w;
        }
    }
    return s0 + s1;
}

// Activations are staged in LDS by the whole block.  Their global loads are
// issued BEFORE the first weight loads (a wave waits for its memory
// operations in issue order, so loads issued later would make the prologue
// wait for the weights), then written to LDS while the weights are in flight.
// XV = float4s per thread: enough for B*K <= 1024*XV.
template <int XV>
__device__ __forceinline__ void issue_x(const GemvArgs &a, float4 (&xr)[XV])
{
    const int n = a.B * a.K;
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int i = (v * K2_BLOCK + threadIdx.x) * 4;
        // unconditional load (clamped address): no branch around it
        xr[v] = *reinterpret_cast<const float4 *>(a.x + (i < n ? i : 0));
    }
}

// Write the staged activations to LDS.  With PRO_NORM the single vector is
// the residual stream h and LDS receives GroupedRMSNorm(h) * gamma: G equal
// contiguous groups, each divided by sqrt(mean of its squares + eps).
template <int XV, int PRO>
__device__ __forceinline__ void finish_x(float *xs, const GemvArgs &a, const float4 (&xr)[XV])
{
    const int n = a.B * a.K;
    if constexpr (PRO == PRO_NORM) {
        __shared__ float red[K2_WAVES_PER_BLOCK][K2_MAX_GROUPS];
        __shared__ float rs[K2_MAX_GROUPS];
        const int G = a.groups, gs = a.K / G;
        float ss[K2_MAX_GROUPS];
#pragma unroll
        for (int g = 0; g < K2_MAX_GROUPS; ++g) ss[g] = 0.f;
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = (v * K2_BLOCK + threadIdx.x) * 4;
            const float4 t = xr[v];
            const float q2 = i < n ? t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w : 0.f;
            const int g = i / gs;   // gs % 4 == 0: a float4 never straddles groups
#pragma unroll
            for (int q = 0; q < K2_MAX_GROUPS; ++q) ss[q] += (q == g) ? q2 : 0.f;
        }
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int g = 0; g < K2_MAX_GROUPS; ++g) {
            if (g < G) {                           // wave-uniform
                const float t = wave_sum(ss[g]);
                if (lane == 0) red[wave][g] = t;
            }
        }
        __syncthreads();
        if (threadIdx.x < G) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < K2_WAVES_PER_BLOCK; ++w) t += red[w][threadIdx.x];
            rs[threadIdx.x] = 1.0f / sqrtf(t / (float)gs + a.eps);
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = (v * K2_BLOCK + threadIdx.x) * 4;
            if (i < n) {
                const float r = rs[i / gs];
                const float4 gm = *reinterpret_cast<const float4 *>(a.gamma + i);
                float4 t = xr[v];
                t.x = t.x * r * gm.x; t.y = t.y * r * gm.y;
                t.z = t.z * r * gm.z; t.w = t.w * r * gm.w;
                *reinterpret_cast<float4 *>(xs + i) = t;
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = (v * K2_BLOCK + threadIdx.x) * 4;
            if (i < n) *reinterpret_cast<float4 *>(xs + i) = xr[v];
        }
    }
    __syncthreads();
}

// Rows of unit `unit` (EPI_SWIGLU: R/2 gate rows followed by the matching
// R/2 up rows).
template <int R, int EPI>
__device__ __forceinline__ void unit_rows(const GemvArgs &a, int64_t unit, int64_t *rows, bool *ok)
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (EPI == EPI_SWIGLU) {
            const int64_t g = unit * (R / 2) + (r % (R / 2));
            ok[r] = g < a.n_out;
            rows[r] = (r < R / 2) ? g : g + a.n_out;
        } else {
            rows[r] = unit * R + r;
            ok[r] = rows[r] < a.N;
        }
    }
}

// Issue the loads of pass p (chunks (p*U + u)*64 + lane, u < U) of R rows.
// Loads are unconditional (out-of-range rows and chunks read a clamped, valid
// address): no branches around the loads, so the compiler tracks exactly how
// many are in flight and waits only for the ones it needs.  The arithmetic
// skips out-of-range chunks, and rows past N are never written.
template <int WDT, int R, int U>
__device__ __forceinline__ void load_pass(const GemvArgs &a, const int64_t *rows, const bool *ok,
                                          int p, int CPR, int lane, k2_u4 (&w)[U][R],
                                          float (&sc)[U][R])
{
    const char *__restrict__ Wb = reinterpret_cast<const char *>(a.W);
    const int64_t row_bytes = (int64_t)CPR * 16;
    const int64_t last_row = (int64_t)a.N - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (p * U + u) * K2_WAVE + lane;
        const int cc = c < CPR ? c : CPR - 1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t rr = rows[r] < last_row ? rows[r] : last_row;
            w[u][r] = __builtin_nontemporal_load(reinterpret_cast<const k2_u4 *>(Wb + rr * row_bytes) + cc);
            if constexpr (WDT == K2_MXFP4) sc[u][r] = e8m0_to_f32(a.S8[rr * CPR + cc]);
        }
    }
}

template <int WDT, int R, int U, int B, int PRO, int EPI, int XV>
__global__ __launch_bounds__(K2_BLOCK) __attribute__((amdgpu_waves_per_eu(3, 8)))
void gemv_kernel(const GemvArgs a)
{
    extern __shared__ float4 lds4[];
    float *xs = reinterpret_cast<float *>(lds4);

    constexpr int EPC = WT<WDT>::EPC;
    const int K = a.K;
    const int CPR = K / EPC;                       // 16-byte chunks per row
    const int passes = (CPR + U * K2_WAVE - 1) / (U * K2_WAVE);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * K2_WAVES_PER_BLOCK;

    // argmax candidate of this thread (EPI_ARGMAX)
    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;

    int64_t unit = (int64_t)blockIdx.x * K2_WAVES_PER_BLOCK + wave;
    int64_t rows[R];
    bool ok[R];
    k2_u4 w[U][R];
    float sc[U][R];
    float4 xr[XV];
    issue_x<XV>(a, xr);                            // activations first ...
    unit_rows<R, EPI>(a, unit, rows, ok);
    // ... then weights (unconditionally: a wave without a unit reads a clamped
    // row it never uses, which keeps the issue path free of branches)
    load_pass<WDT, R, U>(a, rows, ok, 0, CPR, lane, w, sc);
    finish_x<XV, PRO>(xs, a, xr);                  // overlaps the weight loads

#pragma unroll 1
    for (; unit < a.n_units; unit += stride) {
        float acc[B][R];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[b][r] = 0.f;

#pragma unroll 1
        for (int p = 0; p < passes; ++p) {
            if (p > 0) load_pass<WDT, R, U>(a, rows, ok, p, CPR, lane, w, sc);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (p * U + u) * K2_WAVE + lane;
                if (c < CPR) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float *xc = xs + b * K + c * EPC;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float d = chunk_dot<WDT>(w[u][r], xc);
                            if constexpr (WDT == K2_MXFP4) acc[b][r] += d * sc[u][r];
                            else acc[b][r] += d;
                        }
                    }
                }
            }
        }
        // the next unit's first loads fly while this unit is reduced
        int64_t cur_rows[R];
        bool cur_ok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) { cur_rows[r] = rows[r]; cur_ok[r] = ok[r]; }
        const int64_t next = unit + stride;
        unit_rows<R, EPI>(a, next, rows, ok);
        if (next < a.n_units) load_pass<WDT, R, U>(a, rows, ok, 0, CPR, lane, w, sc);  // wave-uniform

#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[b][r] = wave_sum(acc[b][r]);

        if constexpr (WDT == K2_FP8E4M3) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float s = cur_ok[r] ? a.Sf[cur_rows[r]] : 0.f;
#pragma unroll
                for (int b = 0; b < B; ++b) acc[b][r] *= s;
            }
        }

        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int r = 0; r < R / 2; ++r) {
                if (lane == r && cur_ok[r]) {
                    const float g = acc[0][r], u = acc[0][r + R / 2];
                    a.y[cur_rows[r]] = g / (1.0f + expf(-g)) * u;
                }
            }
        } else if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (lane == r && cur_ok[r]) {
                    const float v = acc[0][r];
                    a.y[cur_rows[r]] = v;
                    if (v > best_v || (v == best_v && (int)cur_rows[r] < best_i)) {
                        best_v = v;
                        best_i = (int)cur_rows[r];
                    }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (lane == (b * R + r) % K2_WAVE && cur_ok[r]) {
                        float v = acc[b][r];
                        if (a.residual) v += a.residual[(int64_t)b * a.N + cur_rows[r]];
                        a.y[(int64_t)b * a.N + cur_rows[r]] = v;
                    }
                }
        }
    }

    if constexpr (EPI == EPI_ARGMAX) {
        // per-block candidate; argmax_final_kernel reduces them in block order
        argmax_block(best_v, best_i);
        if (threadIdx.x == 0) {
            a.am.part_v[blockIdx.x] = best_v;
            a.am.part_i[blockIdx.x] = best_i;
        }
    }
}

// ------------------------------------------------------------------ host --

template <int WDT, int R, int U, int B, int PRO, int EPI, int XV>
static int launch(const GemvArgs &a0, hipStream_t st, int max_blocks)
{
    GemvArgs a = a0;
    const int64_t blocks_needed = (a.n_units + K2_WAVES_PER_BLOCK - 1) / K2_WAVES_PER_BLOCK;
    int blocks = (int)(blocks_needed < max_blocks ? blocks_needed : max_blocks);
    if (blocks < 1) blocks = 1;
    const size_t lds = (size_t)B * a.K * sizeof(float);
    hipLaunchKernelGGL((gemv_kernel<WDT, R, U, B, PRO, EPI, XV>), dim3(blocks), dim3(K2_BLOCK), lds,
                       st, a);
    K2_CHECK_LAUNCH();
    if constexpr (EPI == EPI_ARGMAX) return argmax_final_launch(a.am, blocks, st);
    return K2_OK;
}

// Tile choice.  U = 16-byte chunks per lane loaded in one pass (all of a row
// when it has at most 10 per lane, else the row in equal passes), R = rows
// per wave unit: as many waves as there are rows when the matrix is short
// (more waves in flight), up to R*U loads per lane for tall matrices.
struct TileChoice { int R, U; };

// 16-byte loads in flight per lane that fit the register file without spills
// (the wider the decode, the fewer: 32 E2M1 values per MXFP4 chunk).
static constexpr int load_budget(int wdt)
{
    return wdt == K2_MXFP4 ? 8 : wdt == K2_FP8E4M3 ? 12 : 20;
}

static TileChoice choose_tile(int wdt, int N, int K, int B, int epi)
{
    const int epc = wdt == K2_F32 ? 4 : wdt == K2_BF16 ? 8 : wdt == K2_FP8E4M3 ? 16 : 32;
    const int cpl = (K / epc + K2_WAVE - 1) / K2_WAVE;
    int passes = (cpl + 9) / 10;
    int U = (cpl + passes - 1) / passes;
    static const int us[] = {2, 3, 5, 10};
    for (int u : us) if (u >= U) { U = u; break; }
    // at least one row (two for SwiGLU row pairs) must fit the budget
    const int umax = load_budget(wdt) / (epi == EPI_SWIGLU ? 2 : 1);
    while (U > umax) U = U == 10 ? 5 : U == 5 ? 3 : 2;
    int rmax = load_budget(wdt) / U;            // register budget
    int rn = N / 2560;                          // keep >= ~2560 waves in flight
    int R = 1;
    while (R * 2 <= rmax && R * 2 <= rn && R * 2 <= 8) R *= 2;
    if (B > 1) R = 1;
    if (epi == EPI_SWIGLU && R < 2) R = 2;
    return {R, U};
}

template <int WDT, int B, int PRO, int EPI, int R, int U>
static int gemv_go(GemvArgs a, hipStream_t st)
{
    // only register-feasible tiles are instantiated (choose_tile never asks for others)
    if constexpr (R * U <= load_budget(WDT) && (B == 1 || R == 1) && (EPI != EPI_SWIGLU || R >= 2)) {
        if constexpr (EPI == EPI_SWIGLU) a.n_units = (a.n_out + R / 2 - 1) / (R / 2);
        else a.n_units = (a.N + R - 1) / R;
        // float4 activation loads per thread: exactly ceil(B*K / 1024)
        const int64_t bk = (int64_t)a.B * a.K;
        if (bk <= 3 * 1024) return launch<WDT, R, U, B, PRO, EPI, 3>(a, st, K2_GEMV_MAX_BLOCKS);
        if (bk <= 4 * 1024) return launch<WDT, R, U, B, PRO, EPI, 4>(a, st, K2_GEMV_MAX_BLOCKS);
        if (bk <= 10 * 1024) return launch<WDT, R, U, B, PRO, EPI, 10>(a, st, K2_GEMV_MAX_BLOCKS);
        return launch<WDT, R, U, B, PRO, EPI, K2_MAX_LDS_FLOATS / 1024>(a, st, K2_GEMV_MAX_BLOCKS);
    } else {
        return K2_EUNSUPPORTED;
    }
}

template <int WDT, int B, int PRO, int EPI, int R>
static int gemv_u(GemvArgs a, int U, hipStream_t st)
{
    switch (U) {
    case 2: return gemv_go<WDT, B, PRO, EPI, R, 2>(a, st);
    case 3: return gemv_go<WDT, B, PRO, EPI, R, 3>(a, st);
    case 5: return gemv_go<WDT, B, PRO, EPI, R, 5>(a, st);
    default: return gemv_go<WDT, B, PRO, EPI, R, 10>(a, st);
    }
}

template <int WDT, int B, int PRO, int EPI>
static int gemv_tiled(GemvArgs a, hipStream_t st)
{
    const TileChoice t = choose_tile(WDT, EPI == EPI_SWIGLU ? 2 * a.n_out : a.N, a.K, B, EPI);
    switch (t.R) {
    case 1: if constexpr (EPI != EPI_SWIGLU) return gemv_u<WDT, B, PRO, EPI, 1>(a, t.U, st);
            return gemv_u<WDT, B, PRO, EPI, 2>(a, t.U, st);
    case 2: return gemv_u<WDT, B, PRO, EPI, 2>(a, t.U, st);
    case 4: return gemv_u<WDT, B, PRO, EPI, 4>(a, t.U, st);
    default: return gemv_u<WDT, B, PRO, EPI, 8>(a, t.U, st);
    }
}

// Decode-path and generic dispatch for one weight format.
template <int W>
static int gemv_dispatch_fmt(const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    if (pro == PRO_NONE && epi == EPI_PLAIN) {
        switch (a.B) {
        case 1: return gemv_tiled<W, 1, PRO_NONE, EPI_PLAIN>(a, st);
        case 2: return gemv_tiled<W, 2, PRO_NONE, EPI_PLAIN>(a, st);
        case 4: return gemv_tiled<W, 4, PRO_NONE, EPI_PLAIN>(a, st);
        case 8: return gemv_tiled<W, 8, PRO_NONE, EPI_PLAIN>(a, st);
        default: return K2_EUNSUPPORTED;
        }
    }
    if (a.B != 1) return K2_EUNSUPPORTED;
    if (pro == PRO_NORM && epi == EPI_PLAIN) return gemv_tiled<W, 1, PRO_NORM, EPI_PLAIN>(a, st);
    if (pro == PRO_NORM && epi == EPI_SWIGLU) return gemv_tiled<W, 1, PRO_NORM, EPI_SWIGLU>(a, st);
    if (pro == PRO_NORM && epi == EPI_ARGMAX) return gemv_tiled<W, 1, PRO_NORM, EPI_ARGMAX>(a, st);
    return K2_EUNSUPPORTED;
}

}  // namespace k2
