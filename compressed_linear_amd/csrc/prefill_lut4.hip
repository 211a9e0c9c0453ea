// prefill_lut4.hip -- matrix-core prefill kernels for one weight format.
#include "prefill_impl.h"

namespace cl {
template hipError_t launch_prefill_kind<K_LUT4>(const PfArgs&, bool, hipStream_t);
}  // namespace cl
