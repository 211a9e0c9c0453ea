// decode_stream_int8.hip -- batch-1 streaming decode kernels for the INT8 dense format.
#include "decode_stream.h"

namespace cl {
template hipError_t launch_stream_kind<K_INT8>(const StreamArgs&, int, int, int, bool, hipStream_t);
}  // namespace cl
