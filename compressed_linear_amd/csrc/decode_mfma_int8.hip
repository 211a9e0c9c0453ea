// decode_mfma_int8.hip -- matrix-core decode kernels for the INT8 dense format.
#include "decode_mfma.h"

namespace cl {
template hipError_t launch_mfma_kind<K_INT8>(const MfArgs&, bool, hipStream_t);
}  // namespace cl
