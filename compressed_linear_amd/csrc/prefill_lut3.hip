// prefill_lut3.hip -- matrix-core prefill kernels for one weight format.
#include "prefill_impl.h"
#include "prefill_wide.h"

namespace cl {
template hipError_t launch_prefill_kind<K_LUT3>(const PfArgs&, bool, hipStream_t);

// The wide kernel (256 weight rows x 128 activation rows per workgroup).
hipError_t launch_prefill_wide(const PfArgs& a, bool bf16, hipStream_t st) {
  if (a.cptr && a.nsteps_dense > kPfMaxSteps) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(ceil_div(a.ncols, kPwBN) * ceil_div(a.M, kPwBM)));
  if (bf16) hipLaunchKernelGGL(prefill_wide_kernel<true>, grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL(prefill_wide_kernel<false>, grid, dim3(512), 0, st, a);
  return hipGetLastError();
}
}  // namespace cl
