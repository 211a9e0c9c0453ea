// internal.h -- helpers shared by the host translation units of the library.
#pragma once
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

#include "compressed_linear.h"

namespace cl {

// Records a message for cl_last_error() on this thread and returns `st`.
cl_status fail(cl_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Validates the header of a blob and that its sections lie inside it.
cl_status check_blob(const void* blob, const cl_blob_header** out);

}  // namespace cl
