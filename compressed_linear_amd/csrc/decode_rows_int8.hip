// decode_rows_int8.hip -- row-wise decode kernels for the INT8 dense format.
#include "decode_rows.h"

namespace cl {
template hipError_t launch_rows_kind<K_INT8>(const RowArgs&, int, bool, hipStream_t);
}  // namespace cl
