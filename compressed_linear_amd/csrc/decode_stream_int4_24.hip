// decode_stream_int4_24.hip -- batch-1 streaming decode kernels for the INT4 2:4 dense format.
#include "decode_stream.h"

namespace cl {
template hipError_t launch_stream_kind<K_INT4_24>(const StreamArgs&, int, int, int, bool, hipStream_t);
}  // namespace cl
