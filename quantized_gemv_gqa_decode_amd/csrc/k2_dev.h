// k2_dev.h -- device helpers shared by the gfx950 kernels of libk2.
//
// CDNA4 specifics used here: 64-lane wavefronts, 128-bit global loads
// (16 bytes per lane = 1 KiB per wave instruction), the gfx950 hardware
// converters v_cvt_pk_f32_fp8 (OCP E4M3FN -> fp32, two values) and
// v_cvt_scalef32_pk_f32_fp4 (OCP E2M1 -> fp32, two values), and LDS for
// staging activation vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/k2.h"

#define K2_WAVE 64
#define K2_BLOCK 256
#define K2_WAVES_PER_BLOCK (K2_BLOCK / K2_WAVE)

typedef float k2_f2 __attribute__((ext_vector_type(2)));
typedef uint32_t k2_u4 __attribute__((ext_vector_type(4)));

namespace k2 {

// ------------------------------------------------------------- reductions --

// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.  bound_ctrl keeps every lane's own value.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each row of 16 lanes, result in all 16 lanes (4 DPP adds).
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    return v;
}

// Sum over the 64 lanes of the wave, result in every lane: DPP within rows of
// 16, then the four row sums through readlane (uniform scalars).
__device__ __forceinline__ float wave_sum(float v)
{
    v = row16_sum(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum across aligned groups of `W` lanes (W a power of two <= 64), result in
// every lane of the group: DPP inside rows of 16, lane shuffles above.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (W >= 2) v += dpp<0xB1>(v);      // pairs
    if constexpr (W >= 4) v += dpp<0x4E>(v);      // quads
    if constexpr (W >= 8) v += dpp<0x141>(v);     // half rows
    if constexpr (W >= 16) v += dpp<0x140>(v);    // rows
    if constexpr (W >= 32) v += __shfl_xor(v, 16, K2_WAVE);
    if constexpr (W >= 64) v += __shfl_xor(v, 32, K2_WAVE);
    return v;
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations of the wave are outstanding (0 <= n <= 63), without
// waiting on the export or LDS/scalar counters
#define K2_VMCNT(n) (((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

// ---------------------------------------------------------------- codecs --

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two OCP E4M3FN bytes (bytes 0,1 or 2,3 of a dword) -> two fp32.
__device__ __forceinline__ k2_f2 fp8x2_lo(uint32_t u) { return __builtin_amdgcn_cvt_pk_f32_fp8(u, false); }
__device__ __forceinline__ k2_f2 fp8x2_hi(uint32_t u) { return __builtin_amdgcn_cvt_pk_f32_fp8(u, true); }

// Two E2M1 nibbles of byte `SEL` of a dword -> two fp32 (low nibble first).
template <int SEL>
__device__ __forceinline__ k2_f2 fp4x2(uint32_t u)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, SEL);
}

// Low nibble of u as a two's complement int4, divided by 16 (exact:
// v_cvt_off_f32_i4); the Q4S block scale carries the factor 16 back.
__device__ __forceinline__ float q4s_off(uint32_t u) { return __builtin_amdgcn_cvt_off_f32_i4((int)u); }

// E8M0 scale byte -> 2^(b - 127) as fp32 (b = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b)
{
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448; the
// sign bit of the input is kept.
__device__ __forceinline__ uint8_t f32_to_e4m3(float t)
{
    uint32_t sign = (__float_as_uint(t) >> 31) << 7;
    float a = fabsf(t);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7E;
    } else if (a < 0.015625f) {                    // below 2^-6: subnormal step 2^-9
        float q = rintf(a * 512.0f);               // exact scaling, RNE
        code = (uint32_t)q;                        // 8 means 2^-6 = exponent 1, mantissa 0
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // a in [2^e, 2^(e+1))
        float q = rintf(ldexpf(a, 3 - e));         // in [8, 16]
        uint32_t qi = (uint32_t)q;
        if (qi == 16) { e += 1; qi = 8; }
        code = ((uint32_t)(e + 7) << 3) | (qi - 8);
        if (code > 0x7E) code = 0x7E;
    }
    return (uint8_t)(code | sign);
}

// fp32 -> E2M1 code (4 bits), round to nearest even, saturating at +-6; sign kept.
__device__ __forceinline__ uint32_t f32_to_e2m1(float t)
{
    uint32_t sign = (__float_as_uint(t) >> 31) << 3;
    float a = fabsf(t);
    uint32_t code;
    if (a >= 6.0f) {
        code = 7;
    } else if (a < 1.0f) {                         // step 0.5 (subnormal + 1.0)
        code = (uint32_t)rintf(a * 2.0f);          // 0 -> 0, 1 -> 0.5, 2 -> 1.0 (= 0b010)
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // 0, 1 or 2
        uint32_t q = (uint32_t)rintf(ldexpf(a, 1 - e));          // in [2, 4]
        if (q == 4) { e += 1; q = 2; }
        code = ((uint32_t)(e + 1) << 1) | (q - 2);
    }
    return code | sign;
}

// ------------------------------------------------- device-scope accesses --
// Data handed between blocks of ONE grid (the persistent step kernel) may be
// produced and consumed on different XCDs, whose L2 caches are not coherent
// with each other.  Loads and stores with the sc1 (device scope) cache
// policy are performed at device scope; a plain load could return a stale
// line from the reader's L2.

// raw buffer resource over [p, p + 2 GiB): base, no stride, 32-bit words
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k2_rsrc(const void *p)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7FFFFFFF,
                                             0x00020000);
}

constexpr int K2_SC1 = 16;                   // buffer cache-policy bit: sc1

// base must be the same for every lane of the wave (a buffer resource is
// scalar); off = per-lane offset in floats
__device__ __forceinline__ float4 coh_load4(const float *base, int off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(k2_rsrc(base), off * 4, 0, K2_SC1);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}

// base[off .. off + 4) = v at device scope (a vector store with the sc1
// policy); base wave-uniform, off per lane, in floats
__device__ __forceinline__ void coh_store4(float *base, int off, float4 v)
{
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 d = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(d, k2_rsrc(base), off * 4, 0, K2_SC1);
}

__device__ __forceinline__ float coh_load(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int coh_load_i(const int *p)
{
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void coh_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void coh_store_i(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// load / store selected at compile time: COH = device scope, else plain
// base[off .. off + 4): base wave-uniform, off per lane
template <bool COH>
__device__ __forceinline__ float4 ld4(const float *base, int off)
{
    if constexpr (COH) return coh_load4(base, off);
    else return *reinterpret_cast<const float4 *>(base + off);
}

template <bool COH>
__device__ __forceinline__ float ld1(const float *p)
{
    if constexpr (COH) return coh_load(p);
    else return *p;
}

template <bool COH>
__device__ __forceinline__ void st1(float *p, float v)
{
    if constexpr (COH) coh_store(p, v);
    else *p = v;
}

}  // namespace k2

// ------------------------------------------------------------ host helpers --

#define K2_CHECK_LAUNCH()                                    \
    do {                                                     \
        hipError_t e_ = hipGetLastError();                   \
        if (e_ != hipSuccess) return K2_EHIP;                \
    } while (0)

static inline bool k2_aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
static inline bool k2_ptr_ok(const void *p) { return p != nullptr && k2_aligned16(p); }
static inline hipStream_t k2_stream(void *s) { return (hipStream_t)s; }
static inline size_t k2_align256(size_t n) { return (n + 255) & ~(size_t)255; }
