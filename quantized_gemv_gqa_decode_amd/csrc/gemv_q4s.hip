// gemv_q4s.hip -- GEMV instantiations for Q4S int4 weights (see gemv_impl.h).
#include "gemv_impl.h"

namespace k2 {
int gemv_dispatch_q4s(const GemvArgs &a, int pro, int epi, hipStream_t st)
{
    return gemv_dispatch_fmt<K2_Q4S>(a, pro, epi, st);
}
}  // namespace k2
