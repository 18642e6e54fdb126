// pa_logits.hip -- MXFP4 paged MQA logits on gfx950 [FP4API].
//
// Work unit = (sequence b, 256-token chunk), one wavefront. For each 64-token
// KV block of the chunk that holds visible tokens:
//   1. gather the block through block_table: each lane loads 16 FP4 bytes (32
//      channels = one scale group) of one token and that group's UE8M0 byte;
//   2. S[h][t] = q_h . k_t with v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E2M1,
//      E8M0 scales per 32 channels, fp32 result; head_dim 128 is one MFMA);
//      M rows are heads, N columns are tokens, and the heads of a row tile are
//      laid out so that lane group g ends up holding heads [g*H/4, (g+1)*H/4);
//   3. a 4x4 transpose of (lane group, token tile) with permlane32/16 swaps
//      moves all heads of one token into one lane;
//   4. each lane runs the fp32 fma chain over heads in ascending order,
//      weights[row, h] * S[h][t], and stores its token's logit (64 consecutive
//      tokens per store instruction); tokens past the sequence get -inf.
// Blocks past the sequence are never read; their columns are written as -inf.
#include <math.h>

#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

typedef int i8v __attribute__((ext_vector_type(8)));

constexpr int kLogitsChunk = 256;

struct LogitsParams {
  float* out;
  int64_t out_stride;
  const uint8_t* q;
  const int32_t* sf_q;
  const uint8_t* kv;
  const float* w;
  const int32_t* context_lens;
  const int32_t* block_table;
  int B, max_blocks, max_ctx, nchunks;
};

// 4x4 transpose of (lane group, register): after it, register t of lane group
// g holds what register g of lane group t held.
__device__ __forceinline__ void transpose4(float& r0, float& r1, float& r2, float& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(r0), __float_as_uint(r2), false,
                                            false);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(r1), __float_as_uint(r3), false,
                                            false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = __uint_as_float(c[0]);
  r1 = __uint_as_float(c[1]);
  r2 = __uint_as_float(d[0]);
  r3 = __uint_as_float(d[1]);
}

template <int NN, int H>
__global__ __launch_bounds__(64) void logits_kernel(LogitsParams p) {
  constexpr int D = 128, BS = 64;
  constexpr int NTI = H / 16;  // row tiles per query row
  constexpr int HG = H / 4;    // heads per lane group after the MFMA
  constexpr int ROWB = D / 2;  // FP4 bytes per token
  constexpr int SFB = D / 32;  // scale bytes per token
  constexpr int BLK = BS * (ROWB + SFB);
  const int lane = threadIdx.x, j = lane & 15, g = lane >> 4;
  const int c = blockIdx.x % p.nchunks, b = blockIdx.x / p.nchunks;
  const int L = p.context_lens[b];
  const int t_chunk = c * kLogitsChunk;

  // ---- q operands: A rows are heads; row j of row tile rt holds head
  // HG*(j/4) + 4*rt + j%4, lane group g its channels [32g, 32g+32) ----
  i8v qa[NN][NTI];
  int qs[NN][NTI];
  if (t_chunk < L) {
#pragma unroll
    for (int i = 0; i < NN; ++i)
#pragma unroll
      for (int rt = 0; rt < NTI; ++rt) {
        const int h = HG * (j >> 2) + 4 * rt + (j & 3);
        const size_t row = ((size_t)b * NN + i) * H + h;
        const u4 v = *reinterpret_cast<const u4*>(p.q + row * ROWB + 16 * g);
        qa[i][rt] = i8v{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        qs[i][rt] = (p.sf_q[row] >> (8 * g)) & 0xFF;
      }
  }

#pragma unroll 1
  for (int k = 0; k < kLogitsChunk / BS; ++k) {
    const int t_blk = t_chunk + k * BS;
    if (t_blk >= p.max_ctx) break;
    const int t = t_blk + lane;  // the token this lane stores
    if (t_blk >= L) {
      // no visible token in this block: -inf, nothing is read
#pragma unroll
      for (int i = 0; i < NN; ++i)
        if (t < p.max_ctx) p.out[((size_t)b * NN + i) * p.out_stride + t] = -INFINITY;
      continue;
    }
    const uint8_t* blk = p.kv + (size_t)p.block_table[(size_t)b * p.max_blocks + t_blk / BS] * BLK;
    // ---- k operands for the 4 token tiles: column j is token 16*tau + j ----
    i8v kb[4];
    int ks[4];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const int tok = 16 * tau + j;
      const u4 v = *reinterpret_cast<const u4*>(blk + tok * ROWB + 16 * g);
      kb[tau] = i8v{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      ks[tau] = blk[BS * ROWB + tok * SFB + g];
    }
#pragma unroll
    for (int i = 0; i < NN; ++i) {
      float s[NTI][4][4];  // [rt][tau][e]
#pragma unroll
      for (int rt = 0; rt < NTI; ++rt)
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const f4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              qa[i][rt], kb[tau], f4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, qs[i][rt], 0, ks[tau]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[rt][tau][e] = acc[e];
        }
      // lane (j, g) holds heads HG*g + 4*rt + e of tokens 16*tau + j; transpose so
      // that lane (j, g) holds heads HG*tau + 4*rt + e of token 16*g + j
#pragma unroll
      for (int rt = 0; rt < NTI; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) transpose4(s[rt][0][e], s[rt][1][e], s[rt][2][e], s[rt][3][e]);
      const float* wrow = p.w + ((size_t)b * NN + i) * H;
      float acc = 0.f;
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int rt = 0; rt < NTI; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = fmaf(wrow[HG * tau + 4 * rt + e], s[rt][tau][e], acc);
      if (t < p.max_ctx)
        p.out[((size_t)b * NN + i) * p.out_stride + t] = t < L ? acc : -INFINITY;
    }
  }
}

typedef void (*LogitsFn)(LogitsParams);

template <int NN>
LogitsFn pick_h(int H) {
  if (H == 16) return logits_kernel<NN, 16>;
  if (H == 32) return logits_kernel<NN, 32>;
  if (H == 64) return logits_kernel<NN, 64>;
  return nullptr;
}

LogitsFn pick_logits(int NN, int H) {
  switch (NN) {
    case 1: return pick_h<1>(H);
    case 2: return pick_h<2>(H);
    case 3: return pick_h<3>(H);
    case 4: return pick_h<4>(H);
  }
  return nullptr;
}

}  // namespace pa

using namespace pa;

extern "C" size_t paged_mqa_logits_workspace_size(const pa_logits_args* a) {
  (void)a;
  return 0;
}

extern "C" pa_status paged_mqa_logits(const pa_logits_args* a, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!a) return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: args is NULL");
  if (a->batch < 0 || a->next_n < 1 || a->num_heads < 1 || a->head_dim < 1 ||
      a->block_size < 1 || a->max_blocks_per_seq < 1 || a->num_blocks < 1 ||
      a->max_context_len < 0 || a->sf_vec_size < 1)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: bad sizes");
  if (a->head_dim != 128 || a->sf_vec_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: head_dim must be 128, sf_vec_size 32");
  if (a->block_size != 64) return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: block_size must be 64");
  if (a->next_n > 4) return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: next_n must be 1..4");
  LogitsFn fn = pick_logits(a->next_n, a->num_heads);
  if (!fn) return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: num_heads must be 16, 32 or 64");
  if (a->out_row_stride < a->max_context_len)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: out_row_stride < max_context_len");
  // [FP4API, block_table]: at least round_up(max_context_len, 128) / block_size columns
  if ((int64_t)a->max_blocks_per_seq * a->block_size < round_up(a->max_context_len, 128))
    return fail(PA_ERR_PRECONDITION,
                "paged_mqa_logits: block_table needs round_up(max_context_len, 128) / "
                "block_size columns");
  if (a->batch == 0 || a->max_context_len == 0) return PA_OK;
  if (!a->out || !a->q || !a->sf_q || !a->kv_fused || !a->weights || !a->context_lens ||
      !a->block_table)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: null pointer");
  LogitsParams p;
  p.out = a->out;
  p.out_stride = a->out_row_stride;
  p.q = a->q;
  p.sf_q = a->sf_q;
  p.kv = a->kv_fused;
  p.w = a->weights;
  p.context_lens = a->context_lens;
  p.block_table = a->block_table;
  p.B = a->batch;
  p.max_blocks = a->max_blocks_per_seq;
  p.max_ctx = a->max_context_len;
  p.nchunks = (int)ceil_div(a->max_context_len, kLogitsChunk);
  hipStream_t s = (hipStream_t)stream;
  launch_timed(fn, dim3((unsigned)((int64_t)a->batch * p.nchunks)), dim3(64), s, p);
  return launch_status("paged_mqa_logits kernel");
}
