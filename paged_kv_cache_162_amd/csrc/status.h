// Internal helpers shared by the host manager and the device entry points.
#ifndef PAGEDKV_STATUS_H_
#define PAGEDKV_STATUS_H_

#include <cstdarg>
#include <cstddef>

#include "../../include/pagedkv.h"

namespace pagedkv {

// Record a printf-style message for kv_last_error() and return `code`.
kv_status fail(kv_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Reset the calling thread's message at the start of a public call.
void clear_error();
// Element size in bytes; 0 for an unknown dtype.
size_t dtype_bytes(kv_dtype dt);

}  // namespace pagedkv

#endif  // PAGEDKV_STATUS_H_
