// Internal: thread-local error message behind pa_last_error().
#pragma once

#include "pagedkv.h"

namespace pagedkv {

// Records `msg` (printf-style) as this thread's last error and returns `s`.
pa_status fail(pa_status s, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

}  // namespace pagedkv
