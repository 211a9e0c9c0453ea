// decode_rows_int4.hip -- row-wise decode kernels for the INT4 dense format.
#include "decode_rows.h"

namespace cl {
template hipError_t launch_rows_kind<K_INT4>(const RowArgs&, int, bool, hipStream_t);
}  // namespace cl
