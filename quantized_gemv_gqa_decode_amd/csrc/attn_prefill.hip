// attn_prefill.hip -- the causal GQA attention of a prefill chunk on the
// matrix cores (head_dim 128, bf16 or int8 cache).
//
// Semantics are those of the decode attention ([k2-burn] "Model shape": GQA;
// "Limitations": plain SDPA with the softmax in fp32; "KV cache storage":
// bf16 / symmetric int8 with one scale per position and head): the query of
// chunk row t at position p = pos0 + t attends the cached positions [0, p].
// With many rows per chunk this is a dense contraction, so both products run
// on v_mfma_f32_16x16x32_bf16, flash-attention style:
//
//   * a block (4 waves) owns 64 queries of one kv head g: 64 / rep chunk
//     rows x the rep query heads of g; wave w owns queries 16w .. 16w+15;
//   * the block streams the key positions [0, last position of its rows] in
//     tiles of 64 through LDS: K as bf16 rows whose 16-byte chunks are
//     rotated by the key index (conflict-free operand reads), V transposed
//     ([dim][key], rows padded to 136 bytes); int8 codes are widened to bf16
//     exactly while staging.  The next tile's global loads are in flight
//     while the current one is computed;
//   * S^T = K Q^T per 16-key subtile (A = K rows, B = the wave's queries),
//     so a lane holds one query (column) and 4 keys: the row maximum of the
//     online softmax is a max over the lane's 16 values and two lane swaps;
//   * O^T += V^T P^T with P^T taken from the S^T accumulators as they are
//     (the key order inside a 32-key step is permuted identically on both
//     operands, which a contraction allows);
//   * fp32 operands (the rotated queries, the probabilities) enter as bf16
//     hi + lo pairs (two MFMAs), so ~16 bits of each reach the fp32
//     accumulators; the cache values are exact in bf16; the int8 K scale
//     multiplies the finished score and the V scale the probability.
// MFMA operand layout (16x16x32 bf16): lane l holds A row l % 16 and B
// column l % 16, elements k = 8 (l / 16) + [0, 8); D holds column l % 16,
// rows 4 (l / 16) + [0, 4).
#include "attn_impl.h"

namespace k2 {

typedef short ap_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ap_f32x4 __attribute__((ext_vector_type(4)));

constexpr int AP_HD = 128;
constexpr int AP_KT = 64;                  // keys per tile
constexpr int AP_Q = 64;                   // queries per block
constexpr int AP_VTS = AP_KT * 2 + 8;      // bytes per V^T row in LDS
constexpr int AP_MAX_SPLITS = 64;          // key splits (their per-query weights fill the K tile's LDS)

struct ApArgs {
    const float *q;                        // rotated queries [T][n_qh][128]
    const void *kc, *vc;                   // caches [n_kv][cap][128]
    const float *ks, *vs;                  // int8 scales [n_kv][cap]
    float *out;                            // [T][n_qh][128]
    int n_qh, n_kv, cap, pos0, T;
    float qscale;                          // softmax scale * log2(e)
    // key splits (gridDim.z > 1): unnormalised partials [split][T][n_qh][128],
    // their (max, sum) [split][T][n_qh][2], and one arrival counter per
    // (query block, kv head), zero between launches
    float *part, *part_ml;
    unsigned *cnt;
    // the output as bf16 hi / lo planes [T][n_qh * 128] instead of out (nullable)
    uint16_t *oh, *ol;
};

// out[i .. i+3] = v, or its bf16 hi / lo planes
__device__ __forceinline__ void ap_out4(const ApArgs &a, int64_t i, float4 v)
{
    if (a.oh) {
        const float f[4] = {v.x, v.y, v.z, v.w};
        uint16_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = f32_to_bf16_rne(f[e]);
            l[e] = f32_to_bf16_rne(f[e] - bf16_to_f32(h[e]));
        }
        *reinterpret_cast<uint2 *>(a.oh + i) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        *reinterpret_cast<uint2 *>(a.ol + i) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
    } else {
        *reinterpret_cast<float4 *>(a.out + i) = v;
    }
}

__device__ __forceinline__ float ap_xmax(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// bf16 bits of a signed int8 code (exact)
__device__ __forceinline__ uint32_t ap_i8_bf16(uint32_t word, int byte)
{
    const int c = (int)(int8_t)((word >> (8 * byte)) & 0xFFu);
    return __float_as_uint((float)c) >> 16;
}

__device__ __forceinline__ void ap_split(const float (&v)[8], ap_bf16x8 &hi, ap_bf16x8 &lo)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint16_t h = f32_to_bf16_rne(v[e]);
        hi[e] = (short)h;
        lo[e] = (short)f32_to_bf16_rne(v[e] - bf16_to_f32(h));
    }
}

template <int KVDT, int REP>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const ApArgs a)
{
    constexpr bool I8 = KVDT == K2_I8;
    constexpr int PPB = AP_Q / REP;                       // chunk rows per block
    constexpr int NK = I8 ? 2 : 4;                        // K 16-byte loads per thread per tile
    constexpr int NV = I8 ? 1 : 2;                        // V key-pair items per thread per tile
    __shared__ __align__(16) char k_lds[AP_KT * 256];
    __shared__ __align__(16) char vt_lds[AP_HD * AP_VTS];
    __shared__ float ks_lds[AP_KT], vs_lds[AP_KT];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q4 = lane >> 4, c16 = lane & 15;
    const int g = blockIdx.y, t0 = blockIdx.x * PPB;
    const int z = blockIdx.z, NS = gridDim.z;             // key split of this block, splits

    // this lane's query: the column of its S^T and O^T tiles
    const int qi = wave * 16 + c16;
    int t = t0 + qi / REP;
    const bool qvalid = t < a.T;
    t = qvalid ? t : a.T - 1;
    const int h = g * REP + qi % REP;
    const int qpos = a.pos0 + t;
    const int tlast = (t0 + PPB < a.T ? t0 + PPB : a.T) - 1;
    const int kmax = a.pos0 + tlast;                      // the last key a query of the block sees
    const int ntiles = kmax / AP_KT + 1;
    // this split's tiles [tz0, tz1) (empty for a split past the block's keys)
    const int per = (ntiles + NS - 1) / NS;
    const int tz0 = z * per < ntiles ? z * per : ntiles;
    const int tz1 = tz0 + per < ntiles ? tz0 + per : ntiles;

    // the query as B operand of the 4 k-steps of S^T: dims 32j + 8 q4 + [0, 8)
    ap_bf16x8 qh[4], ql[4];
    {
        const float *qrow = a.q + ((int64_t)t * a.n_qh + h) * AP_HD;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 x0 = *reinterpret_cast<const float4 *>(qrow + 32 * j + 8 * q4);
            const float4 x1 = *reinterpret_cast<const float4 *>(qrow + 32 * j + 8 * q4 + 4);
            const float v[8] = {x0.x * a.qscale, x0.y * a.qscale, x0.z * a.qscale, x0.w * a.qscale,
                                x1.x * a.qscale, x1.y * a.qscale, x1.z * a.qscale, x1.w * a.qscale};
            ap_split(v, qh[j], ql[j]);
        }
    }

    using CT = typename KVT<KVDT>::T;
    const CT *kbase = reinterpret_cast<const CT *>(a.kc) + (int64_t)g * a.cap * AP_HD;
    const CT *vbase = reinterpret_cast<const CT *>(a.vc) + (int64_t)g * a.cap * AP_HD;
    const float *ksb = I8 ? a.ks + (int64_t)g * a.cap : nullptr;
    const float *vsb = I8 ? a.vs + (int64_t)g * a.cap : nullptr;

    // the next tile in registers: K 16-byte chunks, V pairs of keys at one
    // dim group (keys past kmax read key kmax: finite, and masked)
    k2_u4 kr[NK], vr[NV][2];
    float sc = 0.f;
    auto load_tile = [&](int tile) {
        const int kb0 = tile * AP_KT;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = i * 256 + tid;
            const int key = I8 ? c / 8 : c / 16, ch = I8 ? c % 8 : c % 16;
            const int kp = kb0 + key < kmax ? kb0 + key : kmax;
            kr[i] = __builtin_nontemporal_load(
                reinterpret_cast<const k2_u4 *>(kbase + (int64_t)kp * AP_HD + ch * (I8 ? 16 : 8)));
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int it = i * 256 + tid;
            const int kp2 = I8 ? it / 8 : it / 16, dg = I8 ? it % 8 : it % 16;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                int kp = kb0 + 2 * kp2 + s;
                kp = kp < kmax ? kp : kmax;
                vr[i][s] = __builtin_nontemporal_load(
                    reinterpret_cast<const k2_u4 *>(vbase + (int64_t)kp * AP_HD + dg * (I8 ? 16 : 8)));
            }
        }
        if constexpr (I8) {
            if (tid < 2 * AP_KT) {
                int kp = kb0 + (tid % AP_KT);
                kp = kp < kmax ? kp : kmax;
                sc = (tid < AP_KT ? ksb : vsb)[kp];
            }
        }
    };
    // registers -> LDS (bf16; K chunk ch of key r at slot (ch + r) % 16)
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = i * 256 + tid;
            if constexpr (I8) {
                const int key = c / 8, c8 = c % 8;
                const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    k2_u4 o;
                    uint32_t ow[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t word = w[half * 2 + e / 2];
                        const int b0 = (e % 2) * 2;
                        ow[e] = ap_i8_bf16(word, b0) | (ap_i8_bf16(word, b0 + 1) << 16);
                    }
                    o.x = ow[0]; o.y = ow[1]; o.z = ow[2]; o.w = ow[3];
                    const int ch = 2 * c8 + half;
                    *reinterpret_cast<k2_u4 *>(k_lds + key * 256 + ((ch + key) & 15) * 16) = o;
                }
            } else {
                const int key = c / 16, ch = c % 16;
                *reinterpret_cast<k2_u4 *>(k_lds + key * 256 + ((ch + key) & 15) * 16) = kr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int it = i * 256 + tid;
            const int kp2 = I8 ? it / 8 : it / 16, dg = I8 ? it % 8 : it % 16;
            const uint32_t w0[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
            const uint32_t w1[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
            constexpr int ND = I8 ? 16 : 8;
#pragma unroll
            for (int e = 0; e < ND; ++e) {
                uint32_t b0, b1;
                if constexpr (I8) {
                    b0 = ap_i8_bf16(w0[e / 4], e % 4);
                    b1 = ap_i8_bf16(w1[e / 4], e % 4);
                } else {
                    b0 = (w0[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
                    b1 = (w1[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
                }
                const int d = dg * ND + e;
                *reinterpret_cast<uint32_t *>(vt_lds + d * AP_VTS + kp2 * 4) = b0 | (b1 << 16);
            }
        }
        if constexpr (I8) {
            if (tid < 2 * AP_KT) (tid < AP_KT ? ks_lds : vs_lds)[tid % AP_KT] = sc;
        }
    };

    ap_f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = ap_f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    if (tz0 < tz1) load_tile(tz0);
#pragma unroll 1
    for (int tile = tz0; tile < tz1; ++tile) {
        __syncthreads();                                  // every wave is done with the previous tile
        store_tile();
        __syncthreads();
        if (tile + 1 < tz1) load_tile(tile + 1);
        const int kb0 = tile * AP_KT;

        // S^T for the 4 subtiles of 16 keys: s[u][e] is key 16u + 4 q4 + e
        ap_f32x4 s[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s[u] = ap_f32x4{0.f, 0.f, 0.f, 0.f};
            const int key = u * 16 + c16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const ap_bf16x8 kv =
                    *reinterpret_cast<const ap_bf16x8 *>(k_lds + key * 256 + ((4 * j + q4 + key) & 15) * 16);
                s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qh[j], s[u], 0, 0, 0);
                s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ql[j], s[u], 0, 0, 0);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kl = u * 16 + 4 * q4 + e;
                float v = s[u][e];
                if constexpr (I8) v *= ks_lds[kl];
                v = kb0 + kl <= qpos ? v : -INFINITY;
                s[u][e] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = ap_xmax(mx);
        const float mn = fmaxf(m, mx);
        const float corr = k2_exp2(m - mn);               // m = -inf gives 0
        m = mn;
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = k2_exp2(s[u][e] - mn);
                ls += p;
                s[u][e] = p;
            }
        l = l * corr + ls;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dt][e] *= corr;

        // O^T += V^T P^T over two 32-key steps; element e of a lane is key
        // 32 st + 4 q4 + e (e < 4) or 32 st + 16 + 4 q4 + e - 4 (e >= 4)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = e < 4 ? s[2 * st][e] : s[2 * st + 1][e - 4];
                if constexpr (I8) pv[e] *= vs_lds[32 * st + (e < 4 ? 0 : 16) + 4 * q4 + (e & 3)];
            }
            ap_bf16x8 ph, pl;
            ap_split(pv, ph, pl);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const char *row = vt_lds + (dt * 16 + c16) * AP_VTS;
                const uint2 lo4 = *reinterpret_cast<const uint2 *>(row + (32 * st + 4 * q4) * 2);
                const uint2 hi4 = *reinterpret_cast<const uint2 *>(row + (32 * st + 16 + 4 * q4) * 2);
                const k2_u4 w = k2_u4{lo4.x, lo4.y, hi4.x, hi4.y};
                const ap_bf16x8 vv = __builtin_bit_cast(ap_bf16x8, w);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, ph, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pl, o[dt], 0, 0, 0);
            }
        }
    }

    // the sum over the lane's 4 key groups, then out = O / l (dims
    // 16 dt + 4 q4 + [0, 4) of the lane's query)
    l = xor16_add(l);
    l = xor32_add(l);
    const int64_t qrow = (int64_t)t * a.n_qh + h;
    if (NS == 1) {
        if (!qvalid) return;
        const float inv = 1.0f / l;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            ap_out4(a, qrow * AP_HD + 4 * q4 + dt * 16,
                    make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv));
        return;
    }

    // key splits: publish this split's partial (device scope), count the
    // block in; the last block of the (query block, kv head) combines
    const int64_t prow = (int64_t)z * a.T * a.n_qh + qrow;
    if (qvalid) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            coh_store4(a.part, (int)(prow * AP_HD + dt * 16 + 4 * q4),
                       make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]));
        if (q4 == 0) {
            coh_store(a.part_ml + prow * 2, m);
            coh_store(a.part_ml + prow * 2 + 1, l);
        }
    }
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);                        // this thread's partial stores completed
    __syncthreads();
    if (tid == 0) {
        unsigned *c = a.cnt + blockIdx.y * gridDim.x + blockIdx.x;
        const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == (unsigned)NS - 1;
        if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;

    // weights of the splits per query, w_z = 2^(m_z - M) / sum_z l_z 2^(m_z - M),
    // in LDS (the K tile's space; every wave is past its last use), then
    // out = sum_z w_z o_z in split order
    float *wz = reinterpret_cast<float *>(k_lds);         // [AP_Q][NS], NS <= AP_MAX_SPLITS
    if (tid < AP_Q) {
        const int tq = t0 + tid / REP, hq = g * REP + tid % REP;
        if (tq < a.T) {
            const int64_t r0 = (int64_t)tq * a.n_qh + hq, stride = (int64_t)a.T * a.n_qh;
            float M = -INFINITY;
            for (int zz = 0; zz < NS; ++zz) M = fmaxf(M, coh_load(a.part_ml + (zz * stride + r0) * 2));
            float L = 0.f;
            for (int zz = 0; zz < NS; ++zz) {
                const float mz = coh_load(a.part_ml + (zz * stride + r0) * 2);
                const float f = mz == -INFINITY ? 0.f : k2_exp2(mz - M);
                wz[tid * NS + zz] = f;
                L += f * coh_load(a.part_ml + (zz * stride + r0) * 2 + 1);
            }
            const float inv = 1.0f / L;
            for (int zz = 0; zz < NS; ++zz) wz[tid * NS + zz] *= inv;
        }
    }
    __syncthreads();
    constexpr int DQ = AP_HD / 4;                         // float4 columns of a query
    for (int it = tid; it < AP_Q * DQ; it += 256) {
        const int qq = it / DQ, dq = it % DQ;
        const int tq = t0 + qq / REP, hq = g * REP + qq % REP;
        if (tq >= a.T) continue;
        const int64_t r0 = (int64_t)tq * a.n_qh + hq, stride = (int64_t)a.T * a.n_qh;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int z0 = 0; z0 < NS; z0 += 8) {
            float4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (z0 + i < NS) v[i] = coh_load4(a.part, (int)(((z0 + i) * stride + r0) * AP_HD + dq * 4));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (z0 + i >= NS) break;
                const float f = wz[qq * NS + z0 + i];
                acc.x += f * v[i].x;
                acc.y += f * v[i].y;
                acc.z += f * v[i].z;
                acc.w += f * v[i].w;
            }
        }
        ap_out4(a, r0 * AP_HD + dq * 4, acc);
    }
}

template <int KVDT>
static int attn_prefill_rep(int rep, const ApArgs &a, int ns, hipStream_t st)
{
    const int ppb = AP_Q / rep;
    const dim3 grid((a.T + ppb - 1) / ppb, a.n_kv, ns);
    switch (rep) {
    case 1: hipLaunchKernelGGL((attn_prefill_kernel<KVDT, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_prefill_kernel<KVDT, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_prefill_kernel<KVDT, 4>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_prefill_kernel<KVDT, 8>), grid, dim3(256), 0, st, a); break;
    default: return K2_EUNSUPPORTED;
    }
    K2_CHECK_LAUNCH();
    return K2_OK;
}

// Key splits: none while the query blocks alone give a block per compute
// unit or the keys are few; else enough for ~2 blocks per compute unit, each
// split at least 4 tiles (256 keys), at most AP_MAX_SPLITS and what the
// workspace holds (max_splits).
static int ap_splits(int T, int rep, int n_kv, int pos0, int max_splits)
{
    const int qb = (T + AP_Q / rep - 1) / (AP_Q / rep);
    const int blocks = qb * n_kv;
    const int ntiles = (pos0 + T - 1) / AP_KT + 1;
    if (blocks >= 256 || ntiles < 8) return 1;
    int ns = (512 + blocks - 1) / blocks;
    ns = ns < ntiles / 4 ? ns : ntiles / 4;
    ns = ns < AP_MAX_SPLITS ? ns : AP_MAX_SPLITS;
    ns = ns < max_splits ? ns : max_splits;
    return ns > 1 ? ns : 1;
}

int attn_prefill_launch(int kvdt, const float *qrot, float *out, const void *kc, const void *vc, const float *ks,
                        const float *vs, int n_qh, int n_kv, int hd, int cap, int pos0, int T, float *part,
                        float *part_ml, int max_splits, unsigned *cnt, uint16_t *oh, uint16_t *ol,
                        hipStream_t st)
{
    if (hd != AP_HD || T < 1 || n_kv < 1 || n_qh % n_kv) return K2_EUNSUPPORTED;
    if (kvdt != K2_BF16 && kvdt != K2_I8) return K2_EUNSUPPORTED;
    if (pos0 < 0 || (int64_t)pos0 + T > cap) return K2_ERANGE;
    const int ns = (part && part_ml && cnt) ? ap_splits(T, n_qh / n_kv, n_kv, pos0, max_splits) : 1;
    ApArgs a{};
    a.oh = oh;
    a.ol = ol;
    a.part = part;
    a.part_ml = part_ml;
    a.cnt = cnt;
    a.q = qrot;
    a.kc = kc;
    a.vc = vc;
    a.ks = ks;
    a.vs = vs;
    a.out = out;
    a.n_qh = n_qh;
    a.n_kv = n_kv;
    a.cap = cap;
    a.pos0 = pos0;
    a.T = T;
    a.qscale = K2_LOG2E / sqrtf((float)hd);
    return kvdt == K2_I8 ? attn_prefill_rep<K2_I8>(n_qh / n_kv, a, ns, st)
                         : attn_prefill_rep<K2_BF16>(n_qh / n_kv, a, ns, st);
}

}  // namespace k2
