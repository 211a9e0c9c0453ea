// prefill_lut3.hip -- matrix-core prefill for the 3-bit LUT format.
#include "prefill_wide.h"

namespace cl {
// The wide kernel (256 weight rows x 128 activation rows per workgroup).
hipError_t launch_prefill_wide(const PfArgs& a, bool bf16, hipStream_t st) {
  if (a.cptr && a.nsteps_dense > kPfMaxSteps) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(ceil_div(a.ncols, kPwBN) * ceil_div(a.M, kPwBM)));
  if (bf16) hipLaunchKernelGGL(prefill_wide_kernel<true>, grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL(prefill_wide_kernel<false>, grid, dim3(512), 0, st, a);
  return hipGetLastError();
}
}  // namespace cl
