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
template <> struct WT<K2_Q4S>     { static constexpr int EPC = 32; };

// Layout of activations staged in LDS.  A 16-byte weight chunk holds EPC
// consecutive elements; lane c of a wave works on chunk c and needs EPC/4
// float4s of x.  Stored linearly, lane c would read at a stride of 4*EPC
// bytes (8-way LDS bank conflicts for MXFP4).  Instead float4 j of chunk c
// is stored at float4 slot j*S + c ("planes" of S float4s): a wave's read of
// plane j is 64 consecutive 16-byte words, and an odd S spreads the EPC/4
// writes of one chunk over distinct banks.  One vector takes EPC*S floats.
__host__ __device__ constexpr int xs_plane(int cpr) { return cpr | 1; }

template <int EPC>
__device__ __forceinline__ int xs_offset(int k, int S)
{
    return (((k % EPC) >> 2) * S + k / EPC) * 4 + (k & 3);
}

template <int I>
__device__ __forceinline__ uint32_t word(const k2_u4 &w)
{
    if constexpr (I == 0) return w.x;
    else if constexpr (I == 1) return w.y;
    else if constexpr (I == 2) return w.z;
    else return w.w;
}

// The 4 weights of plane J (elements 4J..4J+3) of a 16-byte chunk, decoded
// (MXFP4 without its block scale).
template <int WDT, int J>
__device__ __forceinline__ float4 plane_w(const k2_u4 &w)
{
    if constexpr (WDT == K2_F32) {
        return make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                           __uint_as_float(w.w));
    } else if constexpr (WDT == K2_BF16) {
        const uint32_t a = word<2 * J>(w), b = word<2 * J + 1>(w);
        return make_float4(bf16_lo(a), bf16_hi(a), bf16_lo(b), bf16_hi(b));
    } else if constexpr (WDT == K2_FP8E4M3) {
        const uint32_t u = word<J>(w);
        const k2_f2 lo = fp8x2_lo(u), hi = fp8x2_hi(u);
        return make_float4(lo.x, lo.y, hi.x, hi.y);
    } else if constexpr (WDT == K2_MXFP4) {
        // byte m of the chunk holds elements 2m (low nibble) and 2m+1
        const uint32_t u = word<J / 2>(w);
        const k2_f2 v0 = fp4x2<2 * (J % 2)>(u), v1 = fp4x2<2 * (J % 2) + 1>(u);
        return make_float4(v0.x, v0.y, v1.x, v1.y);
    } else {  // Q4S: same nibble order; two's complement int4 -> code / 16
        const uint32_t u = word<J / 2>(w) >> (16 * (J % 2));
        return make_float4(q4s_off(u), q4s_off(u >> 4), q4s_off(u >> 8), q4s_off(u >> 12));
    }
}

// s[b][r] += dot(chunk of row r, chunk of token b) for R rows that share the
// same activation chunk, nb <= B tokens.  Plane-major: one float4 of x per
// token and 4 decoded weights per row are live at a time.  xc: float4 0 of
// the chunk of token 0 in LDS; P: plane stride (floats); TS: token stride.
template <int WDT, int R, int B, int J = 0>
__device__ __forceinline__ void dot_planes(const k2_u4 (&w)[R], const float *__restrict__ xc, int P,
                                           int TS, int nb, float (&s)[B][R])
{
    if constexpr (J < WT<WDT>::EPC / 4) {
        float4 xv[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (b < nb) xv[b] = *reinterpret_cast<const float4 *>(xc + b * TS + J * P);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float4 wv = plane_w<WDT, J>(w[r]);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (b < nb) {
                    s[b][r] = fmaf(wv.x, xv[b].x, s[b][r]);
                    s[b][r] = fmaf(wv.y, xv[b].y, s[b][r]);
                    s[b][r] = fmaf(wv.z, xv[b].z, s[b][r]);
                    s[b][r] = fmaf(wv.w, xv[b].w, s[b][r]);
                }
            }
        }
        dot_planes<WDT, R, B, J + 1>(w, xc, P, TS, nb, s);
    }
}

// One 16-byte chunk per row into acc: MXFP4 applies each row's block scale
// to its partial sum; the other formats accumulate directly (fp8 row scales
// are applied once per row at the end).
template <int WDT, int R, int B>
__device__ __forceinline__ void chunk_rows(const k2_u4 (&w)[R], const float (&sc)[R],
                                           const float *__restrict__ xc, int P, int TS, int nb,
                                           float (&acc)[B][R])
{
    if constexpr (WDT == K2_MXFP4 || WDT == K2_Q4S) {
        float part[B][R];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) part[b][r] = 0.f;
        dot_planes<WDT, R, B>(w, xc, P, TS, nb, part);
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[b][r] = fmaf(part[b][r], sc[r], acc[b][r]);
    } else {
        dot_planes<WDT, R, B>(w, xc, P, TS, nb, acc);
    }
}

// Activations are staged in LDS by the whole block.  Their global loads are
// issued BEFORE the first weight loads (a wave waits for its memory
// operations in issue order, so loads issued later would make the prologue
// wait for the weights), then written to LDS while the weights are in flight.
// XV = float4s per thread: enough for B*K <= 1024*XV.
// COH: x was written by other blocks of the same grid (device-scope loads).
// PRO_NORM: gamma's matching float4s too (gr), for the same reason.
template <int XV, bool COH = false>
__device__ __forceinline__ void issue_x(const GemvArgs &a, float4 (&xr)[XV])
{
    const int n = a.B * a.K;
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int i = (v * K2_BLOCK + threadIdx.x) * 4;
        // unconditional load (clamped address): no branch around it
        xr[v] = ld4<COH>(a.x, i < n ? i : 0);
    }
}
template <int XV>
__device__ __forceinline__ void issue_gamma(const GemvArgs &a, float4 (&gr)[XV])
{
#pragma unroll
    for (int v = 0; v < XV; ++v) {
        const int i = (v * K2_BLOCK + threadIdx.x) * 4;
        gr[v] = *reinterpret_cast<const float4 *>(a.gamma + (i < a.K ? i : 0));
    }
}

// Block barrier for data exchanged through LDS only: it waits for this
// wave's LDS operations, not for its global loads (the weights in flight
// stay in flight; __syncthreads' fence would wait for them).
__device__ __forceinline__ void gemv_lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0); vmcnt, expcnt not waited
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Write the staged activations to LDS.  With PRO_NORM the single vector is
// the residual stream h and LDS receives GroupedRMSNorm(h) * gamma: G equal
// contiguous groups, each divided by sqrt(mean of its squares + eps).
template <int XV, int PRO, int EPC, bool EG>
__device__ __forceinline__ void finish_x(float *xs, const GemvArgs &a, const float4 (&xr)[XV],
                                         const float4 (&gr)[XV], int S)
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
        // (with gamma already in registers the norm need not wait for the
        // weights in flight: barriers on the LDS exchange only)
        if constexpr (EG) gemv_lds_barrier(); else __syncthreads();
        if (threadIdx.x < G) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < K2_WAVES_PER_BLOCK; ++w) t += red[w][threadIdx.x];
            rs[threadIdx.x] = 1.0f / sqrtf(t / (float)gs + a.eps);
        }
        if constexpr (EG) gemv_lds_barrier(); else __syncthreads();
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = (v * K2_BLOCK + threadIdx.x) * 4;
            if (i < n) {
                const float r = rs[i / gs];
                const float4 gm = EG ? gr[v] : *reinterpret_cast<const float4 *>(a.gamma + i);
                float4 t = xr[v];
                t.x = t.x * r * gm.x; t.y = t.y * r * gm.y;
                t.z = t.z * r * gm.z; t.w = t.w * r * gm.w;
                *reinterpret_cast<float4 *>(xs + xs_offset<EPC>(i, S)) = t;   // B == 1
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = (v * K2_BLOCK + threadIdx.x) * 4;
            if (i < n) {
                const int b = i / a.K, k = i - b * a.K;
                *reinterpret_cast<float4 *>(xs + b * EPC * S + xs_offset<EPC>(k, S)) = xr[v];
            }
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
            // Q4S: one scale per two chunks; x16 undoes the code / 16 of the decode
            if constexpr (WDT == K2_Q4S) sc[u][r] = 16.0f * a.Sf[rr * (CPR / 2) + cc / 2];
        }
    }
}

// Rows of `unit` and its pass-0 loads (issued now, consumed by gemv_units).
template <int WDT, int R, int U, int EPI>
__device__ __forceinline__ void gemv_prefetch(const GemvArgs &a, int64_t unit, int64_t (&rows)[R],
                                              bool (&ok)[R], k2_u4 (&w)[U][R], float (&sc)[U][R])
{
    constexpr int EPC = WT<WDT>::EPC;
    unit_rows<R, EPI>(a, unit, rows, ok);
    load_pass<WDT, R, U>(a, rows, ok, 0, a.K / EPC, threadIdx.x & 63, w, sc);
}

// The unit loop of one wave, starting at `unit` whose pass-0 loads are in
// rows/ok/w/sc; activations staged in xs (plane stride S).  COH: outputs are
// stored at device scope (read by other blocks of the same grid).
template <int WDT, int R, int U, int B, int EPI, bool COH>
__device__ __forceinline__ void gemv_units(const GemvArgs &a, const float *xs, int S, int64_t unit,
                                           int64_t stride, int64_t (&rows)[R], bool (&ok)[R],
                                           k2_u4 (&w)[U][R], float (&sc)[U][R], float &best_v,
                                           int &best_i)
{
    constexpr int EPC = WT<WDT>::EPC;
    const int CPR = a.K / EPC;                     // 16-byte chunks per row
    const int passes = (CPR + U * K2_WAVE - 1) / (U * K2_WAVE);
    const int lane = threadIdx.x & 63;
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
                if (c < CPR) chunk_rows<WDT, R, B>(w[u], sc[u], xs + c * 4, 4 * S, EPC * S, B, acc);
            }
        }
        // the next unit's first loads fly while this unit is reduced
        int64_t cur_rows[R];
        bool cur_ok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) { cur_rows[r] = rows[r]; cur_ok[r] = ok[r]; }
        const int64_t next = unit + stride;
        unit_rows<R, EPI>(a, next, rows, ok);
        if (next < a.n_units) load_pass<WDT, R, U>(a, rows, ok, 0, CPR, lane, w, sc);  // uniform

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
                    const float gt = acc[0][r], up = acc[0][r + R / 2];
                    st1<COH>(a.y + cur_rows[r], gt / (1.0f + expf(-gt)) * up);
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
                        st1<COH>(a.y + (int64_t)b * a.N + cur_rows[r], v);
                    }
                }
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
    const int S = xs_plane(a.K / EPC);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t stride = (int64_t)gridDim.x * K2_WAVES_PER_BLOCK;
    const int64_t unit = (int64_t)blockIdx.x * K2_WAVES_PER_BLOCK + wave;

    float best_v = -INFINITY;                      // argmax candidate (EPI_ARGMAX)
    int best_i = 0x7FFFFFFF;
    int64_t rows[R];
    bool ok[R];
    k2_u4 w[U][R];
    float sc[U][R];
    float4 xr[XV];
    // gamma with the activations (so that the norm prologue runs while the
    // weights are in flight) where the registers allow: R * U <= 10 chunks
    // per lane, and not for the lm_head, whose many units per wave make the
    // prologue a small part and which loses a wave per SIMD to the registers
    // (MXFP4 84.4 against 86.3 us; gate/up 10.7 against 11.65 us with it)
    constexpr bool EG = PRO == PRO_NORM && R * U <= 10 && EPI != EPI_ARGMAX;
    float4 gr[XV];
    issue_x<XV>(a, xr);                            // activations (and gamma) first ...
    if constexpr (EG) issue_gamma<XV>(a, gr);
    // (kept ahead of the weight loads: the scheduler would otherwise sink the
    // gamma loads below them, and its use would then wait for every weight)
    __builtin_amdgcn_sched_barrier(0);
    // ... then weights (unconditionally: a wave without a unit reads a clamped
    // row it never uses, which keeps the issue path free of branches)
    gemv_prefetch<WDT, R, U, EPI>(a, unit, rows, ok, w, sc);
    finish_x<XV, PRO, EPC, EG>(xs, a, xr, gr, S);  // overlaps the weight loads
    gemv_units<WDT, R, U, B, EPI, false>(a, xs, S, unit, stride, rows, ok, w, sc, best_v, best_i);

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
    constexpr int EPC = WT<WDT>::EPC;
    const size_t lds = (size_t)B * EPC * xs_plane(a.K / EPC) * sizeof(float);
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
    return (wdt == K2_MXFP4 || wdt == K2_Q4S) ? 8 : wdt == K2_FP8E4M3 ? 12 : 20;
}

static TileChoice choose_tile(int wdt, int N, int K, int B, int epi)
{
    const int epc = wdt == K2_F32 ? 4 : wdt == K2_BF16 ? 8 : wdt == K2_FP8E4M3 ? 16 : 32;  // MXFP4, Q4S 32
    const int cpl = (K / epc + K2_WAVE - 1) / K2_WAVE;
    // rows of more than 5 chunks per lane stream in passes of at most 5:
    // measured on the bf16 down projection (2560 x 10240) R1 U5 (4 passes)
    // 11.7 us against 12.5 us for R1 U10 (2 passes) and 19 us for one pass
    // of 20, on the bf16 O projection (2560 x 4096) 6.5 us against 7.35, on
    // the fp8 down projection 9.1 us against 10.4
    // 4-bit rows stream in passes of at most 3 (MXFP4 down 2560 x 10240:
    // 8.5 us in 2 passes against 8.9 in one of 5; Q4S 9.1 against 9.3)
    const int upass = (wdt == K2_MXFP4 || wdt == K2_Q4S) ? 3 : 5;
    int passes = (cpl + upass - 1) / upass;
    int U = (cpl + passes - 1) / passes;
    static const int us[] = {2, 3, 5, 10};
    for (int u : us) if (u >= U) { U = u; break; }
    // at least one row (two for SwiGLU row pairs) must fit the budget
    const int umax = load_budget(wdt) / (epi == EPI_SWIGLU ? 2 : 1);
    while (U > umax) U = U == 10 ? 5 : U == 5 ? 3 : 2;
    int rmax = load_budget(wdt) / U;            // register budget
    int rn = N / 2560;                          // keep >= ~2560 waves in flight
    // a tall fp8 matrix of short rows (the lm_head, 250624 x 2560: 3 chunks
    // per lane) streams faster with two rows per wave than four (110 us
    // against 119)
    if (wdt == K2_FP8E4M3 && N >= 65536 && rmax > 2) rmax = 2;
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
