// gemv_mxfp4.hip -- GEMV instantiations for mxfp4 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace k2 {
int gemv_dispatch_mxfp4(const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    return gemv_dispatch_fmt<K2_MXFP4>(a, pro, epi, st);
}
}  // namespace k2
