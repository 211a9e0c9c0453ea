// prefill_lr.hip -- matrix-core kernels of the low-rank prologue t = x' L.
#include "prefill_impl.h"

namespace cl {
template hipError_t launch_prefill_kind<K_DENSE16>(const PfArgs&, bool, hipStream_t);
}  // namespace cl
