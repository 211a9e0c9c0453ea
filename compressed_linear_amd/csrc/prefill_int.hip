// prefill_int.hip -- matrix-core prefill kernels for the integer weight formats.
#include "prefill_impl.h"

namespace cl {
template hipError_t launch_prefill_kind<K_INT4>(const PfArgs&, bool, hipStream_t);
template hipError_t launch_prefill_kind<K_INT4_24>(const PfArgs&, bool, hipStream_t);
template hipError_t launch_prefill_kind<K_INT8>(const PfArgs&, bool, hipStream_t);
}  // namespace cl
