// decode_lut3.hip -- decode kernels for the LUT3 dense format.
#include "decode_impl.h"

namespace cl {
template hipError_t launch_decode_kind<K_LUT3>(const DecodeArgs&, bool, hipStream_t);
}  // namespace cl
