// pa_common.hip -- thread-local error state of libpa.
#include <string.h>

#include "pa_host.hpp"

namespace pa {

static thread_local char g_err[512] = "";

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

pa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return pa::g_err; }
