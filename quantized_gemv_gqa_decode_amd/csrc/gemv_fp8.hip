// gemv_fp8.hip -- GEMV instantiations for fp8 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace k2 {
int gemv_dispatch_fp8(const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    return gemv_dispatch_fmt<K2_FP8E4M3>(a, pro, epi, st);
}
}  // namespace k2
