// pa_probe.hip -- a streaming-read probe for benchmarks: the HBM read rate a
// plain kernel reaches on this device, the practical ceiling the attention
// kernels' bandwidth is read against.
#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread

// Every thread reads 16-byte pieces i, i + stride, ... (kProbeUnroll of them
// issued before any is used) and folds them into an xor; each workgroup
// writes one word so the loads are live.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u4* __restrict__ src,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t grid,
                                   void* stream) {
  if (bytes < 0 || (bytes & 15) || grid < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_read_probe: bytes must be a multiple of 16, grid >= 1");
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return fail(PA_ERR_INVALID_ARG, "pa_read_probe: null pointer");
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0,
                     (hipStream_t)stream, (const u4*)src, bytes / 16, sink);
  return launch_status("pa_read_probe kernel");
}
