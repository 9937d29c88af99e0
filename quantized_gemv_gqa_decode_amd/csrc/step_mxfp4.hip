// step_mxfp4.hip -- persistent decode-step kernels for mxfp4 weights (one
// translation unit per weight format, so the instantiations build in parallel).
#include "step_impl.h"

namespace k2 {
int step_dispatch_mxfp4(int kvdt, int hd, int rep, const StepArgs &A, int H, int qd, int inter,
                        int max_blocks, hipStream_t st)
{
    return step_dispatch_t<K2_MXFP4>(kvdt, hd, rep, A, H, qd, inter, max_blocks, st);
}
}  // namespace k2
