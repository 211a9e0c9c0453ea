// decode_rows_lut3.hip -- row-wise decode kernels for the LUT3 dense format.
#include "decode_rows.h"

namespace cl {
template hipError_t launch_rows_kind<K_LUT3>(const RowArgs&, int, bool, hipStream_t);
}  // namespace cl
