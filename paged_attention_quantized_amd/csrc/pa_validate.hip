// pa_validate.hip -- device-side precondition checks enabled by PA_VALIDATE=1
// ("flashinfer.fp4_paged_mqa_logits" API documentation, max_context_len
// parameter: validation of context_lens against max_context_len is optional
// and skipped while a CUDA graph is being captured).
//
// The check kernel reads only context_lens and, for each sequence, the block
// table columns that hold visible tokens (at most ceil(min(L, max_context_len)
// / block_size) of them, all inside the table by the host-checked width), so
// violating inputs are reported before any kernel dereferences them.
#include <stdlib.h>
#include <string.h>

#include "pa_host.hpp"

namespace pa {

// flags[0]: OR of violation bits; flags[1]: smallest violating sequence index.
constexpr int kBadLength = 1, kNullBlock = 2, kBlockRange = 4;

__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ table,
                                                       const int32_t* __restrict__ lens, int B,
                                                       int max_blocks, int max_ctx, int bs,
                                                       int64_t num_blocks, int null_reserved,
                                                       int* flags) {
  const int b = blockIdx.x;
  if (b >= B) return;
  const int L = lens[b];
  int bad = (L < 0 || L > max_ctx) ? kBadLength : 0;
  const int vis = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int pages = (vis + bs - 1) / bs;  // <= max_blocks (checked on the host)
  for (int j = threadIdx.x; j < pages; j += blockDim.x) {
    const int id = table[(size_t)b * max_blocks + j];
    if (id < 0 || (int64_t)id >= num_blocks) bad |= kBlockRange;
    else if (id == 0 && null_reserved) bad |= kNullBlock;
  }
  if (bad) {
    atomicOr(&flags[0], bad);
    atomicMin(&flags[1], b);
  }
}

bool validation_requested() {
  const char* v = getenv("PA_VALIDATE");
  return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
}

pa_status validate_tables(const char* who, const int32_t* table, const int32_t* lens, int B,
                          int max_blocks, int max_ctx, int bs, int64_t num_blocks,
                          bool null_reserved, int* flags, hipStream_t s) {
  if (!validation_requested() || B <= 0) return PA_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: hipStreamIsCapturing failed", who);
  if (cs != hipStreamCaptureStatusNone) return PA_OK;  // skipped while capturing
  if (hipMemsetAsync(flags, 0, sizeof(int), s) != hipSuccess ||
      hipMemsetAsync(flags + 1, 0x7F, sizeof(int), s) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: validation flags could not be cleared", who);
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)B), dim3(256), 0, s, table, lens, B,
                     max_blocks, max_ctx, bs, num_blocks, null_reserved ? 1 : 0, flags);
  pa_status st = launch_status("validation kernel");
  if (st != PA_OK) return st;
  int host[2] = {0, 0};
  if (hipMemcpyAsync(host, flags, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: validation flags could not be read", who);
  if (host[0] == 0) return PA_OK;
  return fail(PA_ERR_PRECONDITION,
              "%s: PA_VALIDATE: sequence %d (first of the violating ones):%s%s%s", who, host[1],
              (host[0] & kBadLength) ? " context_lens outside [0, max_context_len]" : "",
              (host[0] & kBlockRange) ? " a visible page's block id outside [0, num_blocks)" : "",
              (host[0] & kNullBlock) ? " a visible page mapped to the null block 0" : "");
}

}  // namespace pa
