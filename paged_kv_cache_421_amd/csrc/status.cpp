#include "status.h"

#include <cstdarg>
#include <cstdio>

namespace pagedkv {

static thread_local char g_last_error[512] = "";

pa_status fail(pa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace pagedkv

extern "C" const char* pa_last_error(void) { return pagedkv::g_last_error; }

#ifdef PA_DEBUG
extern "C" const char* pa_version(void) { return "pagedkv 0.1 (gfx950, PA_DEBUG)"; }
#else
extern "C" const char* pa_version(void) { return "pagedkv 0.1 (gfx950)"; }
#endif
