// attn_o.hip -- launcher of the attention + O projection launch
// (attn_o_impl.h) for the shapes it is instantiated for: head_dim 128,
// 4 query heads per kv head, O input <= 4096 floats.
#include "attn_o_impl.h"

namespace k2 {

// ------------------------------------------------ attention + O, one launch --

// O rows per wave; chunks per lane cover one 4096-wide row of each format in
// one pass (f32 16, bf16 8, fp8 4, MXFP4 and Q4S 2)
constexpr int AO_R = 2;        // 1 measured slower (19.1 against 17.6 us at 776 positions)
template <int WDT> struct AoTile { static constexpr int U = 4096 / (K2_WAVE * WT<WDT>::EPC); };

template <int WDT, int KVDT>
static int attn_o_go(const AttnOArgs &f0, hipStream_t st)
{
    constexpr int HD = 128, REP = 4, U = AoTile<WDT>::U, EPC = WT<WDT>::EPC;
    constexpr int WPB = ATT_NT / K2_WAVE;
    AttnOArgs f = f0;
    f.o.n_units = (f.o.N + AO_R - 1) / AO_R;
    const int no = (int)((f.o.n_units + WPB - 1) / WPB);
    size_t lds = attn_stream_lds_floats<KVDT, HD, REP>();
    const size_t lc = combine_lds_floats<REP, ATT_NT>();
    const size_t lo = (size_t)EPC * xs_plane(f.o.K / EPC);
    lds = lds > lc ? lds : lc;
    lds = lds > lo ? lds : lo;
    if (lds * sizeof(float) > 160 * 1024) return K2_EUNSUPPORTED;
    auto kern = attn_o_kernel<WDT, KVDT, HD, REP, AO_R, U>;
    // blocks of this launch one compute unit holds at once (LDS, waves,
    // registers), asked once per instantiation
    static const int per_cu = [&] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(kern), ATT_NT,
                                                         lds * sizeof(float)) != hipSuccess)
            n = 1;
        return n < 1 ? 1 : n;
    }();
    const int cus = device_cus();
    if (cus <= 0) return K2_EUNSUPPORTED;
    // only when both roles fit the chip at once (else the two kernels).  A
    // device position's split count is not known here: the grid's split
    // extent is cut to what fits beside the O blocks, and the kernel takes
    // longer ranges per block where the position needs more splits than that
    if (f.at.d_pos) {
        const int room = (cus * per_cu - no) / f.at.n_kv;
        if (room < 1) return K2_EUNSUPPORTED;
        f.at.S = f.at.S < room ? f.at.S : room;
    }
    f.na = f.at.S * f.at.n_kv;
    if (f.na + no > cus * per_cu) return K2_EUNSUPPORTED;
    hipLaunchKernelGGL(kern, dim3(f.na + no), dim3(ATT_NT), lds * sizeof(float), st, f);
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
// per-block stage timestamps of the last attention + O launch (trace builds)
extern "C" int k2_attn_o_trace_read(unsigned long long *out, int n)
{
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(k2::k2_attn_trace), sizeof(unsigned long long) * n) ==
                   hipSuccess ? 0 : -4;
}
#endif
