// Thread-local error string and process-wide options of libpa (host only, no HIP).
#pragma once

#include <cstdint>

#include "pa.h"

namespace pa {
// Record a printf-style message for pa_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int64_t option(int32_t id);
}  // namespace pa
