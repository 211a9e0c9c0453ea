// decode_mfma_int4.hip -- matrix-core decode kernels for the INT4 dense format.
#include "decode_mfma.h"

namespace cl {
template hipError_t launch_mfma_kind<K_INT4>(const MfArgs&, bool, hipStream_t);
}  // namespace cl
