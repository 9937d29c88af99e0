// step_bf16.hip -- persistent decode-step kernels for bf16 weights (one
// translation unit per weight format, so the instantiations build in parallel).
#include "step_impl.h"

namespace k2 {
int step_dispatch_bf16(int kvdt, int hd, int rep, const StepArgs &A, int H, int qd, int inter,
                        int max_blocks, hipStream_t st)
{
    return step_dispatch_t<K2_BF16>(kvdt, hd, rep, A, H, qd, inter, max_blocks, st);
}
}  // namespace k2

#ifdef K2_STEP_TRACE
extern "C" int k2_step_trace_read(unsigned long long *out, int n)
{
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(k2::k2_step_trace), sizeof(unsigned long long) * n) ==
                   hipSuccess ? 0 : -4;
}
#endif
