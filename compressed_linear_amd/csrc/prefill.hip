// prefill.hip -- large-M forward.
#include <hip/hip_runtime.h>

#include "layer.h"

namespace cl {

// Row blocks of 32 through the decode kernels (first version of the path).
hipError_t launch_prefill(const Layer& L, int M, const void* x, float* y, hipStream_t stream) {
  const int ldx = (x == L.xprep) ? L.Kx : L.h.K;
  for (int m0 = 0; m0 < M; m0 += kMaxDecodeM) {
    const int mb = M - m0 < kMaxDecodeM ? M - m0 : kMaxDecodeM;
    const void* xb = static_cast<const uint16_t*>(x) + (size_t)m0 * ldx;
    Layer Lb = L;
    if (x == L.xprep) Lb.xprep = const_cast<uint16_t*>(static_cast<const uint16_t*>(xb));
    hipError_t e = hipSuccess;
    if (L.h.lr != CL_LR_NONE) e = launch_lowrank_prologue(Lb, mb, xb, stream);
    if (e == hipSuccess) e = launch_decode(Lb, mb, xb, y + (size_t)m0 * L.h.N, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cl
