// decode_stream_lut4.hip -- batch-1 streaming decode kernels for the LUT4 dense format.
#include "decode_stream.h"

namespace cl {
template hipError_t launch_stream_kind<K_LUT4>(const StreamArgs&, int, int, int, bool, hipStream_t);
}  // namespace cl
