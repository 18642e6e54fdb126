// pa_topk.hip -- top-k token selection over MQA logits on gfx950: the step
// that turns the indexer's per-token logits [FP4API] into the selected token
// ids of each query row that the sparse route consumes [RELOC, Investigation:
// the selected token ids; Upstream check: top-k].
//
// One workgroup of 1024 threads per logits row. Every logit of the row's
// visible tokens is mapped to a 32-bit key that orders like the value (+0
// and -0 alike, NaN below every number); a radix select over four 8-bit
// digits, most significant first, finds the k-th largest key T and how many
// tokens of key T still fit. Then each thread owns a contiguous run of token
// ids, and two block-wide prefix sums -- over tokens of key T (the lowest ids
// win the ties) and over selected tokens -- give every selected token its
// position: ids come out in ascending order.
#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

struct TopkParams {
  int32_t* sel;
  const void* logits;
  int64_t stride;
  const int32_t* lens;
  int fmt, next_n, k;
};

__device__ __forceinline__ float logit_at(const TopkParams& p, int64_t i) {
  if (p.fmt == PA_LOGITS_F16)
    return (float)__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(p.logits)[i]);
  if (p.fmt == PA_LOGITS_BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p.logits)[i] << 16);
  return static_cast<const float*>(p.logits)[i];
}

// Key whose unsigned order is the selection order of the values: larger value
// larger key, +0 and -0 the same key, NaN the smallest key (0).
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of x over the workgroup (thread order); *total gets
// the sum. `ws` holds kTopkWaves ints of LDS.
__device__ __forceinline__ int block_excl_scan(int x, int* ws, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) ws[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const int w = ws[i];
    before += i < wv ? w : 0;
    all += w;
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ int hist[256];
  __shared__ int scan_ws[kTopkWaves];
  __shared__ int pick[2];  // digit, tokens above it
  const int r = blockIdx.x, tid = threadIdx.x;
  const int k = p.k;
  int32_t* out = p.sel + (size_t)r * k;
  const int64_t base = (int64_t)r * p.stride;
  int L = p.lens[r / p.next_n];
  L = L < 0 ? 0 : (L > p.stride ? (int)p.stride : L);
  if (L <= k) {  // every token is selected
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < L ? j : -1;
    return;
  }
  // ---- radix select of the k-th largest key ----
  uint32_t prefix = 0u, mask = 0u;
  int remaining = k;  // tokens still to take at or below the current prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < L; t += kTopkThreads) {
      const uint32_t key = order_key(logit_at(p, base + t));
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255 - 4l .. 252 - 4l (descending); the first digit
      // at which the count from the top reaches `remaining` is the k-th's
      int c[4], s = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * tid - e];
        s += c[e];
      }
      const int above = wave_incl_scan(s) - s;  // tokens in higher digits
      int run = above, hit = -1, hit_above = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (hit < 0 && run + c[e] >= remaining) {
          hit = 255 - 4 * tid - e;
          hit_above = run;
        }
        run += c[e];
      }
      const uint64_t any = __builtin_amdgcn_ballot_w64(hit >= 0);
      const int first = __builtin_ctzll(any);
      if (tid == first) {
        pick[0] = hit;
        pick[1] = hit_above;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    mask |= 255u << shift;
    remaining -= pick[1];
    __syncthreads();
  }
  // ---- positions: thread tid owns token ids [t0, t1) ----
  const int per = (L + kTopkThreads - 1) / kTopkThreads;
  const int t0 = min(L, tid * per), t1 = min(L, t0 + per);
  int n_gt = 0, n_eq = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = order_key(logit_at(p, base + t));
    n_gt += key > prefix;
    n_eq += key == prefix;
  }
  int total;
  const int eq_before = block_excl_scan(n_eq, scan_ws, &total);
  // tokens of key T are taken lowest id first: `remaining` of them
  const int eq_take = max(0, min(n_eq, remaining - eq_before));
  const int pos0 = block_excl_scan(n_gt + eq_take, scan_ws, &total);
  int pos = pos0, eq_seen = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = order_key(logit_at(p, base + t));
    bool take = key > prefix;
    if (key == prefix) take = eq_seen++ < eq_take;
    if (take) out[pos++] = t;
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_topk_select(const pa_topk_args* a, void* stream) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "pa_topk_select: args is NULL");
  if (a->batch < 0 || a->next_n < 1 || a->k < 1 || a->logits_row_stride < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_topk_select: bad sizes");
  if (a->logits_format != PA_LOGITS_F32 && a->logits_format != PA_LOGITS_F16 &&
      a->logits_format != PA_LOGITS_BF16)
    return fail(PA_ERR_INVALID_ARG, "pa_topk_select: unknown logits_format");
  const int64_t rows = (int64_t)a->batch * a->next_n;
  if (rows == 0) return PA_OK;
  if (rows > 0x7FFFFFFF) return fail(PA_ERR_UNSUPPORTED, "pa_topk_select: too many rows");
  if (!a->sel || !a->logits || !a->context_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_topk_select: null pointer");
  TopkParams p;
  p.sel = a->sel;
  p.logits = a->logits;
  p.stride = a->logits_row_stride;
  p.lens = a->context_lens;
  p.fmt = a->logits_format;
  p.next_n = a->next_n;
  p.k = a->k;
  launch_timed(topk_kernel, dim3((unsigned)rows), dim3(kTopkThreads), (hipStream_t)stream, p);
  return launch_status("pa_topk_select kernel");
}
