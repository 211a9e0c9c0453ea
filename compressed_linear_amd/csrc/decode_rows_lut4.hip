// decode_rows_lut4.hip -- row-wise decode kernels for the LUT4 dense format.
#include "decode_rows.h"

namespace cl {
template hipError_t launch_rows_kind<K_LUT4>(const RowArgs&, int, bool, hipStream_t);
}  // namespace cl
