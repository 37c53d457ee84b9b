// Error reporting and version string for libpagedattn.
#include "status.h"

#include <cstdlib>
#include <cstring>

namespace pa {

static thread_local char g_last_error[512] = "no error";

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bool check_mode() {
  const char* v = std::getenv("PA_CHECK");
  return v != nullptr && std::strcmp(v, "1") == 0;
}

}  // namespace pa

extern "C" const char* pa_version(void) { return "libpagedattn 0.1 (gfx950)"; }

extern "C" const char* pa_last_error(void) { return pa::g_last_error; }
