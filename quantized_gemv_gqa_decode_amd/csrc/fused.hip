// fused.hip -- launcher of the fused QKV + attention + O layer kernel
// (fused_impl.h) for the shapes it is instantiated for.
#include "fused_impl.h"

namespace k2 {

__global__ void zero_words_kernel(unsigned *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

int fused_zero_sync(unsigned *sync, int words, hipStream_t st)
{
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256 < 64 ? (words + 255) / 256 : 64),
                       dim3(256), 0, st, sync, words);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

template <int WDT, int KVDT, int HD, int REP, int XVQ, int XVO>
static int fused_go(FusedArgs f, hipStream_t st)
{
    using TL = FusedTiles<WDT>;
    constexpr int EPC = WT<WDT>::EPC;
    f.q.n_units = (f.q.N + TL::RQ - 1) / TL::RQ;
    f.o.n_units = (f.o.N + TL::RO - 1) / TL::RO;
    f.nq = (int)((f.q.n_units + K2_WAVES_PER_BLOCK - 1) / K2_WAVES_PER_BLOCK);
    f.na = f.at.S * f.at.n_kv;
    const int no = (int)((f.o.n_units + K2_WAVES_PER_BLOCK - 1) / K2_WAVES_PER_BLOCK);
    size_t lds = (size_t)EPC * xs_plane(f.q.K / EPC);
    const size_t lo = (size_t)EPC * xs_plane(f.o.K / EPC);
    const size_t la = attn_stream_lds_floats<KVDT, HD, REP, StreamLean>();
    const size_t lc = combine_lds_floats<REP, K2_BLOCK>();
    lds = lds > lo ? lds : lo;
    lds = lds > la ? lds : la;
    lds = lds > lc ? lds : lc;
    hipLaunchKernelGGL((fused_qao_kernel<WDT, KVDT, HD, REP, XVQ, XVO>), dim3(f.nq + f.na + no),
                       dim3(K2_BLOCK), lds * sizeof(float), st, f);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

template <int WDT>
static int fused_kv(int kvdt, const FusedArgs &f, hipStream_t st)
{
    switch (kvdt) {
    case K2_F32: return fused_go<WDT, K2_F32, 128, 4, 3, 4>(f, st);
    case K2_BF16: return fused_go<WDT, K2_BF16, 128, 4, 3, 4>(f, st);
    case K2_I8: return fused_go<WDT, K2_I8, 128, 4, 3, 4>(f, st);
    default: return K2_EUNSUPPORTED;
    }
}

// Shapes with a fused kernel: head_dim 128, 4 query heads per kv head, QKV
// input <= 3072 floats, O input <= 4096 floats (3 and 4 staged float4s per
// thread), at most FUSE_MAX_KV kv heads.  K2_EUNSUPPORTED otherwise (nothing
// enqueued).
bool fused_ok(int hd, int rep, int n_kv, int hidden, int n_qh_hd)
{
    const int qkv_rows = n_qh_hd + 2 * n_kv * hd;        // QKV blocks of 8 rows (RQ = 2) get flags
    return hd == 128 && rep == 4 && n_kv <= FUSE_MAX_KV && hidden <= 3 * 1024 && n_qh_hd <= 4 * 1024 &&
           qkv_rows <= FUSE_MAX_QKV_BLOCKS * K2_WAVES_PER_BLOCK * 2;
}

int fused_qao_launch(int wdt, int kvdt, const FusedArgs &f, hipStream_t st)
{
    switch (wdt) {
    case K2_F32: return fused_kv<K2_F32>(kvdt, f, st);
    case K2_BF16: return fused_kv<K2_BF16>(kvdt, f, st);
    case K2_FP8E4M3: return fused_kv<K2_FP8E4M3>(kvdt, f, st);
    case K2_MXFP4: return fused_kv<K2_MXFP4>(kvdt, f, st);
    default: return K2_EUNSUPPORTED;
    }
}

// ------------------------------------------------ attention + O, one launch --

// O rows per wave; chunks per lane cover one 4096-wide row of each format in
// one pass (f32 16, bf16 8, fp8 4, MXFP4 and Q4S 2)
constexpr int AO_R = 2;
template <int WDT> struct AoTile { static constexpr int U = 4096 / (K2_WAVE * WT<WDT>::EPC); };

template <int WDT, int KVDT>
static int attn_o_go(const AttnOArgs &f0, hipStream_t st)
{
    constexpr int HD = 128, REP = 4, U = AoTile<WDT>::U, EPC = WT<WDT>::EPC;
    constexpr int WPB = ATT_NT / K2_WAVE;
    AttnOArgs f = f0;
    f.o.n_units = (f.o.N + AO_R - 1) / AO_R;
    f.na = f.at.S * f.at.n_kv;
    const int no = (int)((f.o.n_units + WPB - 1) / WPB);
    const int cus = device_cus();
    if (cus <= 0 || f.na + no > cus) return K2_EUNSUPPORTED;
    size_t lds = attn_stream_lds_floats<KVDT, HD, REP>();
    const size_t lc = combine_lds_floats<REP, ATT_NT>();
    const size_t lo = (size_t)EPC * xs_plane(f.o.K / EPC);
    lds = lds > lc ? lds : lc;
    lds = lds > lo ? lds : lo;
    if (lds * sizeof(float) > 160 * 1024) return K2_EUNSUPPORTED;
    hipLaunchKernelGGL((attn_o_kernel<WDT, KVDT, HD, REP, AO_R, U>), dim3(f.na + no), dim3(ATT_NT),
                       lds * sizeof(float), st, f);
    K2_CHECK_LAUNCH();
    return K2_OK;
}

template <int WDT>
static int attn_o_kv(int kvdt, const AttnOArgs &f, hipStream_t st)
{
    switch (kvdt) {
    case K2_F32: return attn_o_go<WDT, K2_F32>(f, st);
    case K2_BF16: return attn_o_go<WDT, K2_BF16>(f, st);
    case K2_I8: return attn_o_go<WDT, K2_I8>(f, st);
    default: return K2_EUNSUPPORTED;
    }
}

int attn_o_launch(int wdt, int kvdt, int hd, int rep, const AttnArgs &at, const GemvArgs &o,
                  int32_t *d_err, hipStream_t st)
{
    if (hd != 128 || rep != 4 || o.B != 1 || o.K > 4096 || o.K % 4) return K2_EUNSUPPORTED;
    AttnOArgs f{};
    f.at = at;
    f.o = o;
    f.d_err = d_err;
    switch (wdt) {
    case K2_F32: return attn_o_kv<K2_F32>(kvdt, f, st);
    case K2_BF16: return attn_o_kv<K2_BF16>(kvdt, f, st);
    case K2_FP8E4M3: return attn_o_kv<K2_FP8E4M3>(kvdt, f, st);
    case K2_MXFP4: return attn_o_kv<K2_MXFP4>(kvdt, f, st);
    case K2_Q4S: return attn_o_kv<K2_Q4S>(kvdt, f, st);
    default: return K2_EUNSUPPORTED;
    }
}

}  // namespace k2

#ifdef K2_ATTN_TRACE
extern "C" int k2_fused_trace_read(unsigned long long *out, int n)
{
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(k2::k2_attn_trace), sizeof(unsigned long long) * n) ==
                   hipSuccess ? 0 : -4;
}
#endif
