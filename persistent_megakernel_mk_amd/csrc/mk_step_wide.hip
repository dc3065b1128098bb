// The step kernel for decode steps of more than 8 rows (bf16 weights): the same phases as
// mk_step_kernel, with every weight fragment multiplied against two 8-row groups of activation columns.
// A separate build so that the kernels for up to 8 rows keep their product loop unchanged.
#include "mk_device.h"

extern "C" __global__ void __launch_bounds__(kThreads) mk_step_kernel_wide(StepArgs args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  (void)args;
  step_body<false, kRingWide, true>(smem);
}
