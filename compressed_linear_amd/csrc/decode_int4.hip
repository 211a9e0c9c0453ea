// decode_int4.hip -- decode kernels for the INT4 dense format.
#include "decode_impl.h"

namespace cl {
template hipError_t launch_decode_kind<K_INT4>(const DecodeArgs&, bool, hipStream_t);
}  // namespace cl
