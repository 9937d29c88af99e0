// gemv_bf16.hip -- GEMV instantiations for bf16 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace k2 {
int gemv_dispatch_bf16(const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    return gemv_dispatch_fmt<K2_BF16>(a, pro, epi, st);
}
}  // namespace k2
