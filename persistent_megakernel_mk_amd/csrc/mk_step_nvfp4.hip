// The step kernel for configurations with NVFP4 expert weights: the same phases as mk_step_kernel,
// with NVFP4 items (codes of four fragments and their E4M3 scales) in the weight stream. A separate
// build so that the bf16-only product loop carries no FP4 branch.
#include "mk_device.h"

extern "C" __global__ void __launch_bounds__(kThreads) mk_step_kernel_nvfp4(StepArgs args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  (void)args;
  step_body<true, kRingNvfp4>(smem);
}
