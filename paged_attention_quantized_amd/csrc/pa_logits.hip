// pa_logits.hip -- MXFP4 paged MQA logits on gfx950 [FP4API].
//
// Work unit = (sequence b, 64-token block), one wavefront; a workgroup holds
// four consecutive blocks of one sequence. For a block that holds visible
// tokens:
//   1. gather it through block_table: lane l loads, for token tile tau (32
//      tokens) and K half kh, the 16 FP4 bytes of token 32 tau + l % 32 at
//      channels 64 kh + 32 (l / 32) .. + 32 (one scale group) and that group's
//      UE8M0 byte. All loads are issued before the first MFMA;
//   2. S = q . k with v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1, E8M0
//      scales per 32 channels, fp32 result; head_dim 128 is two MFMAs). A row
//      rho of a 32-row tile is query row 2P + ((rho >> 2) & 1) of row pair P
//      and head 16 ht + 4 (rho >> 3) + (rho & 3) of head tile ht; B columns
//      are the 32 tokens of a token tile. The 32x32 result puts row
//      8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32 in register r of lane
//      l, so lane l holds heads 16 ht .. 16 ht + 15 of its own (query row
//      2P + l / 32, token 32 tau + l % 32), head 16 ht + r in register r: no
//      data moves between lanes;
//   3. each lane continues the fp32 fma chain over those heads in ascending
//      order, weights[row, h] * S[h][t] (weights read four at a time), one
//      head tile after the other; then it stores its logit (32 consecutive
//      tokens of one row per half-wave); tokens past the sequence get -inf.
// Blocks past the sequence are never read; their columns are written as -inf.
#include <math.h>

#include "pa_device.hpp"
#include "pa_host.hpp"

#ifndef LOGITS_NB
#define LOGITS_NB 1
#endif
#ifndef LOGITS_WGW
#define LOGITS_WGW 4
#endif
#ifndef LOGITS_WPE
#define LOGITS_WPE 6
#endif

namespace pa {

typedef int i8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kLogitsBlocks = LOGITS_NB;  // 64-token blocks per wave
constexpr int kLogitsWaves = LOGITS_WGW;  // waves per workgroup
constexpr int kLogitsThreads = 64 * kLogitsWaves;

struct LogitsParams {
  void* out;
  int64_t out_stride;
  const uint8_t* q;
  const int32_t* sf_q;
  const uint8_t* kv;
  const float* w;
  const int32_t* context_lens;
  const int32_t* block_table;
  int B, max_blocks, max_ctx, ngroups;
  int sfi;   // scale tail in the interleaved slot order
  int relu;  // rectifier between each head's dot and its weight
  int epi;   // epilogue type of the head chain: PA_LOGITS_F32 / F16 / BF16
};

// fp32 value rounded to bf16 (nearest even), as an fp32
__device__ __forceinline__ float round_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return x != x ? x : __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// fp32 value rounded to the epilogue type (nearest even), as an fp32
template <int EPI>
__device__ __forceinline__ float epi_round(float x) {
  if constexpr (EPI == PA_LOGITS_F16) return (float)(_Float16)x;
  else if constexpr (EPI == PA_LOGITS_BF16) return round_bf16(x);
  else return x;
}

// One row tile's 16 heads of the weighted head chain of one token, continuing
// acc, heads in ascending order: acc = fma(w_h, A(S_h), acc) in fp32, or with
// a reduced-precision epilogue the weight and A(S_h) rounded to that type and
// every step's result rounded to it too [FP4API, epi_dtype; the page does not
// define the arithmetic: the reading taken is rounding at those three points].
// A is the identity or the rectifier. s[t][e] holds head 4 t + e of the tile,
// wrow the tile's 16 weights (16-byte aligned: read four at a time).
template <int EPI>
__device__ __forceinline__ float head_chain16(const float (&s)[4][4], const float* wrow, bool relu,
                                              float acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const f4 w = *reinterpret_cast<const f4*>(wrow + 4 * t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = s[t][e];
      if (relu) x = x > 0.f ? x : 0.f;
      float f = fmaf(w[e], epi_round<EPI>(x), acc);
      // the fp32 result is a value of its own: the compiler would otherwise
      // fuse the fma and the fp16 conversion into one rounding (v_fma_mix)
      if constexpr (EPI != PA_LOGITS_F32) asm volatile("" : "+v"(f));
      acc = epi_round<EPI>(f);
    }
  }
  return acc;
}

// Keeps a loaded value where it is: the empty asm needs the value in a register
// here, so the compiler can neither sink the load into a later branch nor
// split the loads of a chunk into several waits.
template <typename T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// A workgroup is kLogitsWaves waves over as many consecutive chunks of one
// sequence (4: 2 and 8 measured within a few percent); NB = 64-token KV blocks
// per wave (chunk = 64*NB tokens). The q rows of the sequence are staged once
// per workgroup in LDS.
// OT: output element type (float, _Float16 or __bf16; conversions round to
// nearest even).
template <int NN, int H, int NB, typename OT>
__global__ __launch_bounds__(kLogitsThreads) __attribute__((amdgpu_waves_per_eu(LOGITS_WPE))) void logits_kernel(
    LogitsParams p) {
  constexpr int D = 128, BS = 64;
  constexpr int CH = NB * BS;  // tokens per chunk
  constexpr int NTI = H / 16;  // row tiles per query row
  constexpr int ROWB = D / 2;  // FP4 bytes per token
  constexpr int SFB = D / 32;  // scale bytes per token
  constexpr int BLK = BS * (ROWB + SFB);
  constexpr int QN = NN * H * ROWB / 16;  // 16-byte q pieces of the sequence
  constexpr int T = kLogitsThreads;
  constexpr int QP = (QN + T - 1) / T;           // q pieces per thread
  constexpr int SP = (NN * H + T - 1) / T;       // scale words and weights per thread
  __shared__ __attribute__((aligned(16))) uint8_t qlds[NN * H * ROWB];
  __shared__ int32_t sflds[NN * H];
  __shared__ __attribute__((aligned(16))) float wlds[NN * H];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = blockIdx.x % p.ngroups, b = blockIdx.x / p.ngroups;
  const int L = p.context_lens[b];
  const int t_grp = grp * kLogitsWaves * CH;
  const int t_chunk = t_grp + wave * CH;
  const bool grp_live = t_grp < L;  // some wave of the workgroup reads KV
  // blocks of this chunk inside max_context_len, and those holding visible tokens
  const int nblk = max(0, min(NB, (p.max_ctx - t_chunk + BS - 1) / BS));
  const int nvis = t_chunk < L ? min(nblk, (L - t_chunk + BS - 1) / BS) : 0;
  OT* orow = reinterpret_cast<OT*>(p.out) + (size_t)b * NN * p.out_stride;

  // ---- loads that need only b: this chunk's block-table columns (lane k reads
  // column k, clamped to the last column inside max_context_len), the q rows of
  // the sequence (each thread QP 16-byte pieces), their scales and weights ----
  const int32_t* trow = p.block_table + (size_t)b * p.max_blocks + t_chunk / BS;
  // (a wave with no visible block loads nothing: it only writes -inf columns)
  const int pg_lane = nvis > 0 ? trow[min(lane, nblk - 1)] : 0;
  u4 qv[QP];
  int sfv[SP];
  float wv[SP];
  if (grp_live) {
#pragma unroll
    for (int k = 0; k < QP; ++k)
      if (tid + T * k < QN)
        qv[k] = reinterpret_cast<const u4*>(p.q + (size_t)b * NN * H * ROWB)[tid + T * k];
#pragma unroll
    for (int k = 0; k < SP; ++k)
      if (tid + T * k < NN * H) {
        sfv[k] = p.sf_q[(size_t)b * NN * H + tid + T * k];
        wv[k] = p.w[(size_t)b * NN * H + tid + T * k];
      }
  }

  // ---- the FP4 rows and scale bytes of all blocks of the chunk: piece
  // 2 tau + kh of lane l is token 32 tau + l % 32, channels 64 kh + 32 (l / 32)
  // .. + 32. A block with no visible token takes the chunk's first block: its
  // loads hit lines already in flight and are never used; a chunk with none
  // reads nothing ----
  const int c32 = lane & 31, hw = lane >> 5;
  u4 kraw[NB][4];
  int ks[NB][4];
  if (nvis > 0) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int pg = __builtin_amdgcn_readlane(pg_lane, k < nvis ? k : 0);
      const uint8_t* blk = p.kv + (size_t)pg * BLK;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int tok = 32 * tau + c32;
        // scale slot of the token: token order, or the interleaved order in
        // which slot k holds token (k % SFB) * (BS / SFB) + k / SFB [FP4API,
        // is_kv_sf_interleaved]: token 16 a + c sits in slot SFB c + a
        static_assert(SFB == 4 && BS / SFB == 16, "interleaved slot arithmetic");
        const int slot = p.sfi ? SFB * (tok & 15) + (tok >> 4) : tok;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          kraw[k][2 * tau + kh] = *reinterpret_cast<const u4*>(blk + tok * ROWB + 32 * kh + 16 * hw);
          ks[k][2 * tau + kh] = blk[BS * ROWB + slot * SFB + 2 * kh + hw];
        }
      }
    }
  }

  // columns of blocks with no visible token: -inf
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int t = t_chunk + k * BS + lane;
    if (k >= nvis && k < nblk && t < p.max_ctx)
#pragma unroll
      for (int i = 0; i < NN; ++i) orow[(size_t)i * p.out_stride + t] = (OT)(-INFINITY);
  }
  if (!grp_live) return;  // uniform over the workgroup

  if (grp_live) {
#pragma unroll
    for (int k = 0; k < QP; ++k)
      if (tid + T * k < QN) reinterpret_cast<u4*>(qlds)[tid + T * k] = qv[k];
#pragma unroll
    for (int k = 0; k < SP; ++k)
      if (tid + T * k < NN * H) {
        sflds[tid + T * k] = sfv[k];
        wlds[tid + T * k] = p.epi == PA_LOGITS_F16    ? epi_round<PA_LOGITS_F16>(wv[k])
                            : p.epi == PA_LOGITS_BF16 ? epi_round<PA_LOGITS_BF16>(wv[k])
                                                      : wv[k];
      }
  }
  __syncthreads();
  if (nvis == 0) return;
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      pin(kraw[k][tau]);
      pin(ks[k][tau]);
    }

  // A rows of this lane: rho = l % 32 is query row 2P + ((rho >> 2) & 1) of the
  // row pair and head 16 ht + 4 (rho >> 3) + (rho & 3)
  const int a_s = (c32 >> 2) & 1, a_h = 4 * (c32 >> 3) + (c32 & 3);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (k >= nvis) continue;
#pragma unroll
    for (int P = 0; P < (NN + 1) / 2; ++P) {
      const int row = 2 * P + hw;                  // the query row this lane chains
      const int arow = min(2 * P + a_s, NN - 1);   // the query row of its A rows
      // the weights are staged in LDS already rounded to the epilogue type
      const float* wrow = wlds + min(row, NN - 1) * H;
      float acc[2] = {0.f, 0.f};
#pragma unroll
      for (int ht = 0; ht < NTI; ++ht) {
        const int h = 16 * ht + a_h;
        i8v qa[2];
        int qs[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const u4 v = *reinterpret_cast<const u4*>(qlds + (arow * H + h) * ROWB + 32 * kh + 16 * hw);
          qa[kh] = i8v{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
          qs[kh] = (sflds[arow * H + h] >> (8 * (2 * kh + hw))) & 0xFF;
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          f16v c = {};
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const u4 kv4 = kraw[k][2 * tau + kh];
            const i8v kb = i8v{(int)kv4[0], (int)kv4[1], (int)kv4[2], (int)kv4[3], 0, 0, 0, 0};
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[kh], kb, c, 4, 4, 0, qs[kh], 0,
                                                                 ks[k][2 * tau + kh]);
          }
          // register 4 t + e holds head 16 ht + 4 t + e of this lane's (row, token)
          float sc[4][4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[t][e] = c[4 * t + e];
          if (p.epi == PA_LOGITS_F16)
            acc[tau] = head_chain16<PA_LOGITS_F16>(sc, wrow + 16 * ht, p.relu, acc[tau]);
          else if (p.epi == PA_LOGITS_BF16)
            acc[tau] = head_chain16<PA_LOGITS_BF16>(sc, wrow + 16 * ht, p.relu, acc[tau]);
          else if (p.relu)
            acc[tau] = head_chain16<PA_LOGITS_F32>(sc, wrow + 16 * ht, true, acc[tau]);
          else
            acc[tau] = head_chain16<PA_LOGITS_F32>(sc, wrow + 16 * ht, false, acc[tau]);
        }
      }
      if (row < NN) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const int t = t_chunk + k * BS + 32 * tau + c32;
          if (t < p.max_ctx) orow[(size_t)row * p.out_stride + t] = (OT)(t < L ? acc[tau] : -INFINITY);
        }
      }
    }
  }
}

typedef void (*LogitsFn)(LogitsParams);

template <int NN, int NB, typename OT>
LogitsFn pick_h(int H) {
  if (H == 16) return logits_kernel<NN, 16, NB, OT>;
  if (H == 32) return logits_kernel<NN, 32, NB, OT>;
  if (H == 64) return logits_kernel<NN, 64, NB, OT>;
  return nullptr;
}

template <int NB, typename OT>
LogitsFn pick_nn(int NN, int H) {
  switch (NN) {
    case 1: return pick_h<1, NB, OT>(H);
    case 2: return pick_h<2, NB, OT>(H);
    case 3: return pick_h<3, NB, OT>(H);
    case 4: return pick_h<4, NB, OT>(H);
  }
  return nullptr;
}

template <int NB>
LogitsFn pick_out(int format, int NN, int H) {
  switch (format) {
    case PA_LOGITS_F32: return pick_nn<NB, float>(NN, H);
    case PA_LOGITS_F16: return pick_nn<NB, _Float16>(NN, H);
    case PA_LOGITS_BF16: return pick_nn<NB, __bf16>(NN, H);
  }
  return nullptr;
}

}  // namespace pa

using namespace pa;

// The workspace only holds the PA_VALIDATE flags (unused otherwise: without
// validation NULL, 0 is accepted).
extern "C" size_t paged_mqa_logits_workspace_size(const pa_logits_args* a) {
  (void)a;
  return kValidateBytes;
}

extern "C" pa_status paged_mqa_logits(const pa_logits_args* a, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: args is NULL");
  if (a->batch < 0 || a->next_n < 1 || a->num_heads < 1 || a->head_dim < 1 ||
      a->block_size < 1 || a->max_blocks_per_seq < 1 || a->num_blocks < 1 ||
      a->max_context_len < 0 || a->sf_vec_size < 1)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: bad sizes");
  if (a->head_dim != 128 || a->sf_vec_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: head_dim must be 128, sf_vec_size 32");
  if (a->block_size != 64) return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: block_size must be 64");
  if (a->next_n > 4) return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: next_n must be 1..4");
  if (a->out_format != PA_LOGITS_F32 && a->out_format != PA_LOGITS_F16 &&
      a->out_format != PA_LOGITS_BF16)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: unknown out_format");
  if (a->epi_format != PA_LOGITS_F32 && a->epi_format != PA_LOGITS_F16 &&
      a->epi_format != PA_LOGITS_BF16)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: unknown epi_format");
  if (a->sf_interleaved != 0 && a->sf_interleaved != 1)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: sf_interleaved must be 0 or 1");
  if (a->relu != 0 && a->relu != 1)
    return fail(PA_ERR_INVALID_ARG, "paged_mqa_logits: relu must be 0 or 1");
  LogitsFn fn = pick_out<kLogitsBlocks>(a->out_format, a->next_n, a->num_heads);
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
  hipStream_t s = (hipStream_t)stream;
  if (validation_requested()) {
    if (!workspace || workspace_bytes < kValidateBytes)
      return fail(PA_ERR_WORKSPACE,
                  "paged_mqa_logits: PA_VALIDATE needs paged_mqa_logits_workspace_size() bytes "
                  "of workspace");
    pa_status st = validate_tables("paged_mqa_logits", a->block_table, a->context_lens, a->batch,
                                   a->max_blocks_per_seq, a->max_context_len, a->block_size,
                                   a->num_blocks, false, (int*)workspace, s);
    if (st != PA_OK) return st;
  }
  LogitsParams p;
  p.out = a->out;
  p.out_stride = a->out_row_stride;
  p.q = a->q;
  p.sf_q = a->sf_q;
  p.kv = a->kv_fused;
  p.w = a->weights;
  p.context_lens = a->context_lens;
  p.block_table = a->block_table;
  p.sfi = a->sf_interleaved;
  p.relu = a->relu;
  p.epi = a->epi_format;
  p.B = a->batch;
  p.max_blocks = a->max_blocks_per_seq;
  p.max_ctx = a->max_context_len;
  p.ngroups = (int)ceil_div(a->max_context_len, kLogitsWaves * 64 * kLogitsBlocks);
  launch_timed(fn, dim3((unsigned)((int64_t)a->batch * p.ngroups)), dim3(kLogitsThreads), s, p);
  return launch_status("paged_mqa_logits kernel");
}
