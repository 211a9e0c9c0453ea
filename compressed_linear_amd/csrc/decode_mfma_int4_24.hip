// decode_mfma_int4_24.hip -- matrix-core decode kernels for the INT4 2:4 dense format.
#include "decode_mfma.h"

namespace cl {
template hipError_t launch_mfma_kind<K_INT4_24>(const MfArgs&, bool, hipStream_t);
}  // namespace cl
