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

}  // namespace k2

#ifdef K2_ATTN_TRACE
extern "C" int k2_fused_trace_read(unsigned long long *out, int n)
{
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(k2::k2_attn_trace), sizeof(unsigned long long) * n) ==
                   hipSuccess ? 0 : -4;
}
#endif
