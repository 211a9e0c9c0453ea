// decode_mfma_int8_bm.hip -- matrix-core decode kernels for the INT8 bitmap dense format.
#include "decode_mfma.h"

namespace cl {
template hipError_t launch_mfma_kind<K_INT8_BM>(const MfArgs&, bool, hipStream_t);
}  // namespace cl
