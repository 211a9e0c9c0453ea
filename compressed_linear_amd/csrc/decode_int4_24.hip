// decode_int4_24.hip -- decode kernels for the INT4_24 dense format.
#include "decode_impl.h"

namespace cl {
template hipError_t launch_decode_kind<K_INT4_24>(const DecodeArgs&, bool, hipStream_t);
}  // namespace cl
