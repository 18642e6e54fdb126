// pa_host.hpp -- host-side helpers of libpa: thread-local error reporting and
// argument checks shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/pa.h"

namespace pa {

pa_status fail(pa_status st, const char* fmt, ...);
void clear_error();
pa_status launch_status(const char* what);
void prof_begin(hipStream_t s);  // record the profiling start event, if set
void prof_end(hipStream_t s);    // record the profiling stop event, if set

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

inline int kv_bits(pa_kv_kind k) {
  switch (k) {
    case PA_KV_F16:
    case PA_KV_BF16:
      return 16;
    case PA_KV_E4M3:
    case PA_KV_INT8:
      return 8;
    case PA_KV_INT4:
      return 4;
  }
  return 0;
}

inline bool valid_kind(int k) { return k >= PA_KV_F16 && k <= PA_KV_INT4; }
inline bool valid_mode(int m) { return m >= PA_SCALE_NONE && m <= PA_SCALE_PER_CHANNEL; }

}  // namespace pa
