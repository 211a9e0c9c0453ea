// decode_stream_lut3.hip -- batch-1 streaming decode kernels for the LUT3 dense format.
#include "decode_stream.h"

namespace cl {
template hipError_t launch_stream_kind<K_LUT3>(const StreamArgs&, int, int, int, bool, hipStream_t);
}  // namespace cl
