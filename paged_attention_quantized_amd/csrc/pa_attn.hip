// pa_attn.hip -- paged attention over a quantized KV cache on gfx950.
//
// Work unit = (sequence b, split s, KV head hk), one wavefront. A split covers
// logical tokens [s*S, (s+1)*S) with S fixed from the shapes only, so the
// reduction order never depends on physical block ids [RELOC, Summary].
// Per 32-token chunk the wave
//   1. reads the chunk's page entries (planner, logical order); entries with
//      mask 0 are never read [NULLPAD, Root cause],
//   2. loads K rows (16 B per lane, coalesced) and V rows (each lane owns
//      head_dim/16 consecutive channels of 8 tokens),
//   3. decodes codes to fp16 in registers (exact for E4M3/INT8/INT4) and zeroes
//      V rows of tail tokens by select [NULLPAD, Fix],
//   4. S^T = K Q'^T with v_mfma_f32_16x16x32_f16 (tokens x query rows); the
//      per-channel K scale is folded into Q' = q * k_scale / max|k_scale|,
//      carried as fp16 hi + lo parts [FOLD, Approach],
//   5. online softmax in the exponent base 2 on raw scores (p = 2^((s - m) c)),
//   6. O^T += V^T P^T with the same MFMA (channels x query rows).
// The unit writes (m, l, c) and the unnormalized O; the merge kernel combines
// splits in ascending logical order and applies v_scale / l.
#include <math.h>

#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

struct AttnParams {
  _Float16* out;
  const _Float16* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  f4* ws_ml;     // [units, R] (m_raw, l, c, 0)
  float* ws_o;   // [units, R, D]
  int B, next_n, Hq, Hkv, G, R, bs, max_blocks;
  int split_tokens, nsplit, pages_per_split;
  int k_scale_mode, v_scale_mode, causal;
  float softmax_scale;
};

template <int KIND, int D, int RT, bool HILO>
__global__ __launch_bounds__(64) void attn_split_kernel(AttnParams p) {
  constexpr int BITS = Kv<KIND>::kBits;
  constexpr int RB = D * BITS / 8;   // bytes per (token, head) row
  constexpr int NJ = RB / 64;        // 16-byte K chunks per lane per token
  constexpr int EPC = 128 / BITS;    // elements per 16-byte chunk
  constexpr int KPC = EPC / 8;       // MFMA k-steps (32 channels) per chunk per lane group
  constexpr int KS = D / 32;         // k-steps of QK
  constexpr int DV = D / 16;         // channels each lane owns for V
  constexpr int VB = RB / 16;        // V bytes per lane per token
  constexpr int VDW = VB / 4;
  static_assert(RB % 64 == 0, "row bytes must be a multiple of 64");
  static_assert(NJ * KPC == KS, "k-step bookkeeping");

  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  int unit = blockIdx.x;
  const int hk = unit % p.Hkv;
  unit /= p.Hkv;
  const int s = unit % p.nsplit;
  const int b = unit / p.nsplit;
  const int L = p.context_lens[b];
  const int t_begin = s * p.split_tokens;
  if (t_begin >= L) return;
  const int t_end = min(t_begin + p.split_tokens, L);
  const int32_t* table_row = p.block_table + (size_t)b * p.max_blocks;
  const int first_lblk = t_begin / p.bs;

  // ---- scale constants: fold normalizer for PER_CHANNEL K [FOLD, Approach] ----
  float qk, inv_m = 0.f;
  if constexpr (HILO) {
    float mx = 0.f;
    for (int i = lane; i < p.Hkv * D; i += 64) mx = fmaxf(mx, fabsf(p.k_scale[i]));
    mx = wave_max(mx);
    inv_m = mx > 0.f ? 1.0f / mx : 0.f;
    qk = p.softmax_scale * mx;
  } else {
    qk = p.softmax_scale * (p.k_scale_mode == PA_SCALE_PER_TENSOR ? p.k_scale[0] : 1.0f);
  }
  const float sgn = qk < 0.f ? -1.f : 1.f;
  const float c2 = fabsf(qk) * kLog2e;

  // ---- Q' operands (B of the QK MFMA): lane (n, g) holds row 16*rt+n, the 8
  // channels of k-step ks that lane group g's K chunk provides ----
  h8 qa[RT][KS];
  h8 qb[RT][HILO ? KS : 1];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + n;
    const bool rv = r < p.R;
    const int i = r / p.G, hg = r % p.G;
    const _Float16* qrow = p.q + (((size_t)b * p.next_n + i) * p.Hq + hk * p.G + hg) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int j = ks / KPC, w = ks % KPC;
      const int d0 = (g + 4 * j) * EPC + 8 * w;
      h8 v = {};
      if (rv) v = *reinterpret_cast<const h8*>(qrow + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + run_elem<KIND>(e);
        const float x = (float)v[run_elem<KIND>(e)];
        if constexpr (HILO) {
          const float xf = x * (p.k_scale[hk * D + d] * inv_m) * sgn;
          const _Float16 hi = (_Float16)xf;
          qa[rt][ks][e] = hi;
          qb[rt][ks][e] = (_Float16)(xf - (float)hi);
        } else {
          qa[rt][ks][e] = (_Float16)(x * sgn);
        }
      }
    }
  }

  f4 o[RT][DV];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int q = 0; q < DV; ++q) o[rt][q] = f4{0.f, 0.f, 0.f, 0.f};
  }
  int lim[RT];  // query row 16*rt+n sees tokens t <= lim
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int i = (16 * rt + n) / p.G;
    lim[rt] = p.causal ? (L - p.next_n + i) : 0x7fffffff;
  }

  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
    u4 kraw[2][NJ];
    uint32_t vraw[8][VDW];
    uint32_t tmask[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tt = t0 + 16 * tau;
      const int e_idx = tt / p.bs - first_lblk;
      const PlanEntry en = plan_entry(table_row, L, p.bs, first_lblk, p.pages_per_split, e_idx);
      const int slot0 = tt % p.bs;
      tmask[tau] = (en.mask >> slot0) & 0xFFFFu;
      if (tmask[tau] != 0u) {
        const uint8_t* base = p.k_cache + (((size_t)en.phys * p.bs + slot0) * p.Hkv + hk) * RB;
        const size_t tok_stride = (size_t)p.Hkv * RB;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          kraw[tau][j] = *reinterpret_cast<const u4*>(base + n * tok_stride + 16 * (g + 4 * j));
        const uint8_t* vbase = p.v_cache + (((size_t)en.phys * p.bs + slot0) * p.Hkv + hk) * RB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint8_t* src = vbase + (4 * g + e) * tok_stride + n * VB;
          if constexpr (VDW == 4) {
            u4 x = *reinterpret_cast<const u4*>(src);
#pragma unroll
            for (int k = 0; k < 4; ++k) vraw[4 * tau + e][k] = x[k];
          } else if constexpr (VDW == 2) {
            u2 x = *reinterpret_cast<const u2*>(src);
            vraw[4 * tau + e][0] = x[0];
            vraw[4 * tau + e][1] = x[1];
          } else {
            vraw[4 * tau + e][0] = *reinterpret_cast<const uint32_t*>(src);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) kraw[tau][j] = u4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int k = 0; k < VDW; ++k) vraw[4 * tau + e][k] = 0u;
      }
      // tail tokens: zero their V codes by select so 0 * NaN never happens
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = (tmask[tau] >> (4 * g + e)) & 1u;
#pragma unroll
        for (int k = 0; k < VDW; ++k) vraw[4 * tau + e][k] = ok ? vraw[4 * tau + e][k] : 0u;
      }
    }

    // ---- S^T = K Q'^T ----
    f4 sacc[2][RT];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      h8 kop[KS];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        _Float16 hv[EPC];
        uint32_t wd[4] = {kraw[tau][j][0], kraw[tau][j][1], kraw[tau][j][2], kraw[tau][j][3]};
        decode_run<KIND, 4>(wd, hv);
#pragma unroll
        for (int w = 0; w < KPC; ++w)
#pragma unroll
          for (int e = 0; e < 8; ++e) kop[j * KPC + w][e] = hv[8 * w + e];
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], qa[rt][ks], acc, 0, 0, 0);
          if constexpr (HILO)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], qb[rt][ks], acc, 0, 0, 0);
        }
        sacc[tau][rt] = acc;
      }
    }

    // ---- online softmax (per query row = lane column n) ----
    h8 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = 4 * g + e;
          const int t = t0 + 16 * tau + tk;
          const bool ok = ((tmask[tau] >> tk) & 1u) && t <= lim[rt];
          const float x = ok ? sacc[tau][rt][e] : -INFINITY;
          sv[4 * tau + e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float m_new = fmaxf(m_run[rt], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f((m_run[rt] - m_use) * c2);
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const _Float16 ph = (_Float16)exp2f((sv[k] - m_use) * c2);
        pb[rt][k] = ph;
        psum += (float)ph;
      }
      l_run[rt] = alpha * l_run[rt] + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int q = 0; q < DV; ++q) o[rt][q] *= alpha;
    }

    // ---- O^T += V^T P^T ----
    _Float16 vh[8][DV];
#pragma unroll
    for (int e = 0; e < 8; ++e) decode_run<KIND, VDW>(vraw[e], vh[e]);
#pragma unroll
    for (int q = 0; q < DV; ++q) {
      h8 vop;
#pragma unroll
      for (int e = 0; e < 8; ++e) vop[e] = vh[e][q];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        o[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pb[rt], o[rt][q], 0, 0, 0);
    }
  }

  // ---- write the split's partial state ----
  const size_t u = blockIdx.x;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = l_run[rt];
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    const int r = 16 * rt + n;
    if (r < p.R) {
      if (g == 0) p.ws_ml[u * p.R + r] = f4{m_run[rt], l, c2, 0.f};
      float* orow = p.ws_o + (u * p.R + r) * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float tmp[DV];
#pragma unroll
        for (int q = 0; q < DV; ++q) tmp[run_elem<KIND>(q)] = o[rt][q][e];
#pragma unroll
        for (int k = 0; k < DV; k += 4)
          *reinterpret_cast<f4*>(orow + DV * (4 * g + e) + k) =
              f4{tmp[k], tmp[k + 1], tmp[k + 2], tmp[k + 3]};
      }
    }
  }
}

// Combine the splits of each (b, hk) in ascending logical order [RELOC] and
// apply the V scale and 1/l. A row with no visible token is +0.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int bh = blockIdx.x;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (idx >= p.R * D) return;
  const int r = idx / D, d = idx % D;
  const int L = p.context_lens[b];
  const int ns = (L + p.split_tokens - 1) / p.split_tokens;
  const int i = r / p.G, h = hk * p.G + r % p.G;
  _Float16* dst = p.out + (((size_t)b * p.next_n + i) * p.Hq + h) * D + d;
  float mstar = -INFINITY, c2 = 0.f;
  for (int s = 0; s < ns; ++s) {
    const f4 rec = p.ws_ml[((size_t)(b * p.nsplit + s) * p.Hkv + hk) * p.R + r];
    mstar = fmaxf(mstar, rec[0]);
    c2 = rec[2];
  }
  float l = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t u = (size_t)(b * p.nsplit + s) * p.Hkv + hk;
    const f4 rec = p.ws_ml[u * p.R + r];
    const float w = rec[0] == -INFINITY ? 0.f : exp2f((rec[0] - mstar) * c2);
    l += w * rec[1];
    o += w * p.ws_o[(u * p.R + r) * D + d];
  }
  float val = l > 0.f ? o / l : 0.f;
  if (p.v_scale_mode == PA_SCALE_PER_TENSOR)
    val *= p.v_scale[0];
  else if (p.v_scale_mode == PA_SCALE_PER_CHANNEL)
    val *= p.v_scale[hk * D + d];
  *dst = (_Float16)val;
}

// Planner probe: the entries the attention kernel walks, one thread per entry.
__global__ void plan_dump_kernel(AttnParams p, int entries_per_unit, int32_t* entries) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.nsplit * entries_per_unit;
  if (idx >= total) return;
  const int e = idx % entries_per_unit;
  const int unit = idx / entries_per_unit;
  const int s = unit % p.nsplit, b = unit / p.nsplit;
  const int L = p.context_lens[b];
  const int first_lblk = s * p.split_tokens / p.bs;
  const PlanEntry x = plan_entry(p.block_table + (size_t)b * p.max_blocks, L, p.bs, first_lblk,
                                 p.pages_per_split, e);
  entries[idx * 3 + 0] = x.phys;
  entries[idx * 3 + 1] = x.lblk;
  entries[idx * 3 + 2] = (int32_t)x.mask;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

struct Shape {
  int R, RT, RB, split, nsplit, pages_per_split, entries_per_unit;
  int64_t units;
  size_t ml_bytes, o_bytes;
};

pa_status check_args(const pa_attn_args* a, Shape* sh, bool need_ptrs) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "paged_attn: args is NULL");
  if (a->batch < 0 || a->next_n < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1 ||
      a->max_context_len < 0 || a->max_blocks_per_seq < 1 || a->num_blocks < 1)
    return fail(PA_ERR_INVALID_ARG, "paged_attn: negative or zero size");
  if (a->num_q_heads % a->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "paged_attn: num_q_heads %% num_kv_heads != 0");
  if (!valid_kind(a->kv_kind) || !valid_mode(a->k_scale_mode) || !valid_mode(a->v_scale_mode))
    return fail(PA_ERR_INVALID_ARG, "paged_attn: unknown kv_kind or scale mode");
  if (a->q_dtype != PA_DT_F16) return fail(PA_ERR_UNSUPPORTED, "paged_attn: q_dtype must be F16");
  if (a->kv_kind == PA_KV_BF16) return fail(PA_ERR_UNSUPPORTED, "paged_attn: BF16 KV unsupported");
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: head_dim must be 64, 128 or 256");
  if (a->block_size != 16 && a->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: block_size must be 16 or 32");
  const int rb = a->head_dim * kv_bits(a->kv_kind) / 8;
  if (rb % 64) return fail(PA_ERR_UNSUPPORTED, "paged_attn: head_dim too small for this kv kind");
  if (a->kv_kind == PA_KV_F16 &&
      (a->k_scale_mode != PA_SCALE_NONE || a->v_scale_mode != PA_SCALE_NONE))
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: F16 KV takes no scales");
  if (a->softmax_scale < 0.f || !(a->softmax_scale == a->softmax_scale))
    return fail(PA_ERR_INVALID_ARG, "paged_attn: softmax_scale must be >= 0");
  const int R = a->next_n * (a->num_q_heads / a->num_kv_heads);
  if (R > 64) return fail(PA_ERR_UNSUPPORTED, "paged_attn: next_n * q heads per kv head > 64");
  if ((int64_t)a->max_blocks_per_seq * a->block_size < a->max_context_len)
    return fail(PA_ERR_PRECONDITION,
                "paged_attn: max_blocks_per_seq * block_size < max_context_len");
  if (need_ptrs) {
    if (!a->out || !a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->context_lens)
      return fail(PA_ERR_INVALID_ARG, "paged_attn: null pointer");
    if ((a->k_scale_mode != PA_SCALE_NONE && !a->k_scale) ||
        (a->v_scale_mode != PA_SCALE_NONE && !a->v_scale))
      return fail(PA_ERR_INVALID_ARG, "paged_attn: scale mode set but scale pointer is NULL");
  }
  sh->R = R;
  sh->RT = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  sh->RB = rb;
  // Split size: from shapes only. Enough units to fill the chip several times,
  // but a split long enough that its partial (R x D fp32) stays small against the
  // KV bytes it reads.
  const int64_t work = (int64_t)a->batch * a->num_kv_heads * (int64_t)a->max_context_len;
  int64_t split = round_up(ceil_div(work > 0 ? work : 1, 4096), 32);
  const int64_t min_split = ceil_div((int64_t)R * a->head_dim * 4 * 16, 2 * (int64_t)rb);
  if (split < min_split) split = min_split;
  if (split < 64) split = 64;
  split = round_up(split, 32);
  if (split > 1 << 20) split = 1 << 20;
  sh->split = (int)split;
  sh->nsplit = (int)(a->max_context_len > 0 ? ceil_div(a->max_context_len, split) : 1);
  sh->pages_per_split = sh->split / a->block_size;
  sh->entries_per_unit = (int)round_up(sh->pages_per_split, 8);
  sh->units = (int64_t)a->batch * sh->nsplit * a->num_kv_heads;
  sh->ml_bytes = (size_t)round_up(sh->units * R * 16, 256);
  sh->o_bytes = (size_t)round_up(sh->units * R * a->head_dim * 4, 256);
  return PA_OK;
}

AttnParams make_params(const pa_attn_args* a, const Shape& sh, void* ws) {
  AttnParams p;
  p.out = (_Float16*)a->out;
  p.q = (const _Float16*)a->q;
  p.k_cache = (const uint8_t*)a->k_cache;
  p.v_cache = (const uint8_t*)a->v_cache;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.context_lens = a->context_lens;
  p.ws_ml = (f4*)ws;
  p.ws_o = (float*)((char*)ws + sh.ml_bytes);
  p.B = a->batch;
  p.next_n = a->next_n;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.R = sh.R;
  p.bs = a->block_size;
  p.max_blocks = a->max_blocks_per_seq;
  p.split_tokens = sh.split;
  p.nsplit = sh.nsplit;
  p.pages_per_split = sh.pages_per_split;
  p.k_scale_mode = a->k_scale_mode;
  p.v_scale_mode = a->v_scale_mode;
  p.causal = a->causal ? 1 : 0;
  p.softmax_scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / sqrtf((float)a->head_dim);
  return p;
}

typedef void (*SplitFn)(AttnParams);

template <int KIND, int D>
SplitFn pick_rt(int RT, bool hilo) {
  if (hilo) {
    if constexpr (KIND == PA_KV_F16) return nullptr;
    else {
      if (RT == 1) return attn_split_kernel<KIND, D, 1, true>;
      if (RT == 2) return attn_split_kernel<KIND, D, 2, true>;
      return attn_split_kernel<KIND, D, 4, true>;
    }
  }
  if (RT == 1) return attn_split_kernel<KIND, D, 1, false>;
  if (RT == 2) return attn_split_kernel<KIND, D, 2, false>;
  return attn_split_kernel<KIND, D, 4, false>;
}

template <int KIND>
SplitFn pick_d(int D, int RT, bool hilo) {
  if constexpr (KIND != PA_KV_INT4)
    if (D == 64) return pick_rt<KIND, 64>(RT, hilo);
  if (D == 128) return pick_rt<KIND, 128>(RT, hilo);
  return pick_rt<KIND, 256>(RT, hilo);
}

SplitFn pick_split(int kind, int D, int RT, bool hilo) {
  switch (kind) {
    case PA_KV_F16: return pick_d<PA_KV_F16>(D, RT, hilo);
    case PA_KV_E4M3: return pick_d<PA_KV_E4M3>(D, RT, hilo);
    case PA_KV_INT8: return pick_d<PA_KV_INT8>(D, RT, hilo);
    case PA_KV_INT4: return pick_d<PA_KV_INT4>(D, RT, hilo);
  }
  return nullptr;
}

SplitFn pick_merge(int D) {
  if (D == 64) return attn_merge_kernel<64>;
  if (D == 128) return attn_merge_kernel<128>;
  return attn_merge_kernel<256>;
}

}  // namespace

}  // namespace pa

using namespace pa;

extern "C" size_t paged_attn_workspace_size(const pa_attn_args* a) {
  Shape sh;
  if (check_args(a, &sh, false) != PA_OK) return 0;
  return sh.ml_bytes + sh.o_bytes;
}

extern "C" pa_status paged_attn_fwd(const pa_attn_args* a, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Shape sh;
  pa_status st = check_args(a, &sh, true);
  if (st != PA_OK) return st;
  if (workspace_bytes < sh.ml_bytes + sh.o_bytes || !workspace)
    return fail(PA_ERR_WORKSPACE, "paged_attn: workspace needs %zu bytes, got %zu",
                sh.ml_bytes + sh.o_bytes, workspace_bytes);
  if (a->batch == 0) return PA_OK;
  const bool hilo = a->k_scale_mode == PA_SCALE_PER_CHANNEL;
  SplitFn fn = pick_split(a->kv_kind, a->head_dim, sh.RT, hilo);
  if (!fn) return fail(PA_ERR_UNSUPPORTED, "paged_attn: no kernel for this kind/shape");
  AttnParams p = make_params(a, sh, workspace);
  hipStream_t s = (hipStream_t)stream;
  prof_begin(s);
  hipLaunchKernelGGL(fn, dim3((unsigned)sh.units), dim3(64), 0, s, p);
  prof_end(s);
  if ((st = launch_status("paged_attn split kernel")) != PA_OK) return st;
  hipLaunchKernelGGL(pick_merge(a->head_dim), dim3((unsigned)(a->batch * a->num_kv_heads),
                     (unsigned)ceil_div((int64_t)sh.R * a->head_dim, 256)), dim3(256), 0, s, p);
  return launch_status("paged_attn merge kernel");
}

extern "C" pa_status pa_plan(const pa_attn_args* a, int32_t* entries, int64_t max_entries,
                             int32_t* info, void* stream) {
  Shape sh;
  pa_status st = check_args(a, &sh, false);
  if (st != PA_OK) return st;
  const int64_t total = (int64_t)a->batch * sh.nsplit * sh.entries_per_unit;
  if (info) {
    info[0] = sh.split;
    info[1] = sh.nsplit;
    info[2] = sh.entries_per_unit;
    info[3] = 0;
  }
  if (!entries) {
    if (!info) return fail(PA_ERR_INVALID_ARG, "pa_plan: entries and info both NULL");
    return PA_OK;
  }
  if (max_entries < total) return fail(PA_ERR_WORKSPACE, "pa_plan: needs %lld entries",
                                       (long long)total);
  if (!a->block_table || !a->context_lens) return fail(PA_ERR_INVALID_ARG, "pa_plan: null ptr");
  AttnParams p = make_params(a, sh, nullptr);
  if (total > 0)
    hipLaunchKernelGGL(plan_dump_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                       (hipStream_t)stream, p, sh.entries_per_unit, entries);
  return launch_status("pa_plan kernel");
}
