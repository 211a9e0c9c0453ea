// decode_int8_bm.hip -- decode kernels for the INT8_BM dense format.
#include "decode_impl.h"

namespace cl {
template hipError_t launch_decode_kind<K_INT8_BM>(const DecodeArgs&, bool, hipStream_t);
}  // namespace cl
