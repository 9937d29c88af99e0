// gemv_f32.hip -- GEMV instantiations for f32 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace k2 {
int gemv_dispatch_f32(const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    return gemv_dispatch_fmt<K2_F32>(a, pro, epi, st);
}
}  // namespace k2
