// decode_mfma_lut3.hip -- matrix-core decode kernels for the LUT3 dense format.
#include "decode_mfma.h"

namespace cl {
template hipError_t launch_mfma_kind<K_LUT3>(const MfArgs&, bool, hipStream_t);
}  // namespace cl
