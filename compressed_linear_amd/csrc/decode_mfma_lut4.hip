// decode_mfma_lut4.hip -- matrix-core decode kernels for the LUT4 dense format.
#include "decode_mfma.h"

namespace cl {
template hipError_t launch_mfma_kind<K_LUT4>(const MfArgs&, bool, hipStream_t);
}  // namespace cl
