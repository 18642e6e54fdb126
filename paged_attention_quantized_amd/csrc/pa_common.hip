// pa_common.hip -- thread-local error state of libpa, and device queries.
#include <string.h>

#include <atomic>

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

// Profiling hook: events the dominant kernel of the next calls on this thread
// is launched with (stamped by the kernel's own dispatch).
static thread_local hipEvent_t g_prof_start = nullptr;
static thread_local hipEvent_t g_prof_stop = nullptr;

bool prof_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_prof_start;
  *stop = g_prof_stop;
  return g_prof_start != nullptr;
}

void set_prof_events(void* start, void* stop) {
  g_prof_start = (hipEvent_t)start;
  g_prof_stop = (hipEvent_t)stop;
}

// Compute units of the current device (the persistent grid size), cached per
// device; threads may race to fill an entry, all with the same value.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

pa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return pa::g_err; }

extern "C" pa_status pa_set_profile_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_set_profile_events: give both events or neither");
  pa::set_prof_events(start_event, stop_event);
  return PA_OK;
}
