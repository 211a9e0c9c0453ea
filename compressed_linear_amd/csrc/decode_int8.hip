// decode_int8.hip -- decode kernels for the INT8 dense format.
#include "decode_impl.h"

namespace cl {
template hipError_t launch_decode_kind<K_INT8>(const DecodeArgs&, bool, hipStream_t);
}  // namespace cl
