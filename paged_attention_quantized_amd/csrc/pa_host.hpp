// pa_host.hpp -- host-side helpers of libpa: thread-local error reporting and
// argument checks shared by the entry points.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/pa.h"

namespace pa {

pa_status fail(pa_status st, const char* fmt, ...);
void clear_error();
pa_status launch_status(const char* what);
// Compute units of the current device (persistent grids take one or a few
// workgroups per unit).
int device_cus();
// Profiling events set by pa_set_profile_events (false if none).
bool prof_events(hipEvent_t* start, hipEvent_t* stop);

// Launch a kernel; with profiling events set, through hipExtLaunchKernelGGL so
// that the events carry the kernel's own start and end times.
template <typename F, typename... Args>
void launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (prof_events(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// PA_VALIDATE=1: device check of context_lens against max_context_len and of
// the block ids of visible pages (range, and the null block 0 when it is
// reserved), then a sync; PA_ERR_PRECONDITION names the first violating
// sequence. Skipped (PA_OK) when validation is off or the stream is
// capturing. `flags` is 8 bytes of device scratch.
bool validation_requested();
pa_status validate_tables(const char* who, const int32_t* table, const int32_t* lens, int B,
                          int max_blocks, int max_ctx, int bs, int64_t num_blocks,
                          bool null_reserved, int* flags, hipStream_t s);
constexpr size_t kValidateBytes = 256;  // workspace bytes reserved for the flags

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
