// pa_attn.hpp -- device side of the paged attention kernels (shared by the
// per-KV-kind translation units and the host part in pa_attn.hip). The design
// is described at the top of pa_attn.hip.
#pragma once

#include <math.h>

#include "pa_device.hpp"

namespace pa {

// LDS ring depth: two items in flight while one is computed (measured faster
// than three in flight on the decode, verify and per-channel workloads: the
// first loads return sooner and the HBM queues stay as full)
constexpr int kStages = 3;
constexpr int kStageMax = 32 * 1024;   // bytes per stage (K and V planes)
constexpr int kMaxWaves = 8;           // wavefronts per workgroup
constexpr int kXchBytes = 32 * 1024;   // LDS exchange buffer (ring + exchange = 128 KiB)
constexpr int kMaxNextN = 4096;        // query steps per sequence
constexpr int kMaxRows = 8192;         // query rows per KV head (next_n * q heads per KV head)

// Q' formats of the ring kernel. Per-tensor scales: Q' is q in fp16.
// Per-channel K scales: Q' = q * k_scale / max|k_scale| in fp32, split into an
// fp16 high part and an fp16 remainder, so the folded scale keeps ~22 bits.
//   kQPlain:  one B operand, query row 16 rt + n in column n.
//   kQSplit:  the fold's parts as two B operands, each summed by its own MFMA.
//   kQPacked: (at most 8 query rows per KV head) one B operand carries the
//             high parts of rows 0-7 in columns 0-7 and the remainders in
//             columns 8-15; a rotation by 8 lanes inside each 16-lane row adds
//             the two halves, so one MFMA per k-step does the work of two.
//   kQDup:    (at most 8 rows, per-tensor scales) rows 0-7 in columns 0-7 and
//             again in columns 8-15.
// In the two packed forms (kQPacked, kQDup) lanes n and n + 8 of a 16-lane row
// hold the same scores, and the softmax weights of the P V product travel as
// an fp16 high part (columns 0-7) and an fp16 remainder (columns 8-15) of one
// k = 16 operand; the halves of O and of the row sums are added when a
// partial is written. In the other forms every lane carries both parts of its
// four tokens in one k = 32 operand (high parts in slots 0-3, remainders in
// 4-7) against the V codes repeated in both halves. Either way p keeps ~22
// bits in the products, not fp16's 11.
constexpr int kQPlain = 0, kQSplit = 1, kQPacked = 2, kQDup = 3;
// per-channel fold (hi + lo Q' parts)
__host__ __device__ constexpr bool qf_fold(int qf) { return qf == kQSplit || qf == kQPacked; }
// query rows in columns 0-7, mirrored in 8-15 (P packed into one k = 16 operand)
__host__ __device__ constexpr bool qf_pack(int qf) { return qf == kQPacked || qf == kQDup; }

// The softmax weights are computed as p * 2^kPScale (the exponent offset is
// one subtraction): the largest weight is 2^14 rather than 1, so the fp16
// remainder of small weights stays out of fp16's subnormal range. O and the
// row sums carry the same factor, which cancels in O / l.
constexpr float kPScale = 14.0f;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

struct AttnParams {
  void* out;           // fp16 or bf16 (out_bf16)
  const uint16_t* q;   // fp16 or bf16 bits (q_bf16)
  int q_bf16, out_bf16;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  f4* ws_ml;     // [partials, R] (m_raw, l, c, 0)
  float* ws_o;   // [partials, R, D]
  int* ws_seq;   // [B + 1]: first cost slot of each sequence, then the slot total
  int B, next_n, Hq, Hkv, G, R, bs, max_blocks;
  // query row blocks: rows r = i * G + g are cut into nrb blocks of rpb rows;
  // one run of items per (sequence, row block, head group). nrb = 1 and
  // rpb = R when R <= 32.
  int nrb, rpb;
  int hpu, hgroups, ts, nw, nsub;  // heads per item, head groups, tokens per item, waves, sub-tiles
  int nwg;                         // workgroups of the persistent grid
  int lbs, lts, lhpu;              // log2 of bs, ts, hpu (all powers of two)
  int wgmerge;                     // sub-tile states merged in the workgroup: one partial per head
                                   // (always, when an item has several sub-tiles)
  int run_cost;                    // work split: items a run start costs (drain, q reload, partial)
  int k_scale_mode, v_scale_mode, causal;
  float softmax_scale;
  // selection-driven sparse mode: union plan of each sequence (entry k =
  // {physical block, logical block}, row masks [entries][next_n]); an item is
  // one plan entry and context_lens holds entries * block_size
  const int32_t* sp_entries;
  const uint32_t* sp_masks;
  int sp_cap;
};


// items of one sequence for one head group
__device__ __forceinline__ int seq_stages(const AttnParams& p, int L) {
  return (L + p.ts - 1) >> p.lts;
}

// Tokens row block rb (rows [rb * rpb, min((rb + 1) * rpb, R)), row r being
// step r / G) can see: under the causal rule its last step i sees
// t <= L - next_n + i; all L otherwise (and for a single block).
__device__ __forceinline__ int run_len(const AttnParams& p, int L, int rb) {
  if (!p.causal || p.nrb == 1) return L;
  const int last = (min((rb + 1) * p.rpb, p.R) - 1) / p.G;
  return max(0, min(L, L - p.next_n + last + 1));
}

// step of row block rb's first row
__device__ __forceinline__ int first_step(const AttnParams& p, int rb) {
  return p.nrb == 1 ? 0 : rb * p.rpb / p.G;
}

// The first item at or after cost slot `rel` of a sequence of length L (rel
// below the sequence's cost): its row block, head group and stage, and its
// index among the sequence's items.
__device__ __forceinline__ int locate_slot(const AttnParams& p, int L, int rel, int& rb, int& hg,
                                           int& k);

// items of the run (sequence of length L, row block rb, one head group)
__device__ __forceinline__ int run_stages(const AttnParams& p, int L, int rb) {
  return seq_stages(p, run_len(p, L, rb));
}

__device__ __forceinline__ int locate_slot(const AttnParams& p, int L, int rel, int& rb, int& hg,
                                           int& k) {
  int before = 0, n = run_stages(p, L, 0);
  rb = 0;
  while (rb + 1 < p.nrb) {
    const int c = n > 0 ? p.hgroups * (n + p.run_cost) : 0;
    if (rel < c) break;
    rel -= c;
    before += p.hgroups * n;
    ++rb;
    n = run_stages(p, L, rb);
  }
  hg = rel / (n + p.run_cost);
  k = max(rel % (n + p.run_cost) - p.run_cost, 0);
  return before + hg * n + k;
}

// A sequence's cost-line slots and items over all its row blocks: each run
// with items takes run_cost slots and then one per item, per head group.
__device__ __forceinline__ void seq_cost(const AttnParams& p, int L, int& cost, int& items) {
  cost = 0;
  items = 0;
  for (int rb = 0; rb < p.nrb; ++rb) {
    const int n = run_stages(p, L, rb);
    cost += n > 0 ? p.hgroups * (n + p.run_cost) : 0;
    items += p.hgroups * n;
  }
}

// Position of one item in the (sequence, head group, stage) order; all fields
// are workgroup-uniform.
struct ItemPos {
  int b, L, nst, hg, k, rb;
};

__device__ __forceinline__ void item_next(const AttnParams& p, const int32_t* __restrict__ lens,
                                          ItemPos& it) {
  if (++it.k < it.nst) return;
  it.k = 0;
  if (++it.hg < p.hgroups) return;
  it.hg = 0;
  do {
    if (++it.rb >= p.nrb) {
      it.rb = 0;
      ++it.b;
      it.L = it.b < p.B ? lens[uni(it.b)] : 0;
    }
    it.nst = run_stages(p, it.L, it.rb);
  } while (it.nst == 0 && it.b < p.B);
}

template <int KIND, int D>
struct Geo {
  static constexpr int BITS = Kv<KIND>::kBits;
  static constexpr int RB = D * BITS / 8;   // bytes per (token, head) row
  static constexpr int CPR = RB / 16;       // 16-byte pieces per row
  static constexpr int NJ = RB / 64;        // K pieces per lane per token
  static constexpr int EPC = 128 / BITS;    // elements per 16-byte piece
  static constexpr int KPC = EPC / 8;       // MFMA k-steps (8 channels per lane) per piece
  static constexpr int KS = D / 32;         // k-steps of QK
  static constexpr int DV = D / 16;         // channels each lane owns for V
  static constexpr int VB = RB / 16;        // V bytes per lane per token
  static constexpr int VDW = VB / 4;
  static constexpr int NL = RB / 32;        // ring loads per thread per stage
  static_assert(RB % 64 == 0, "row bytes must be a multiple of 64");
  static_assert(NJ * KPC == KS, "k-step bookkeeping");
  static_assert(VB <= 16 || VB % 16 == 0, "V bytes per lane");
};

// Workgroup-wide stage loads (the prefill kernel, whose waves all read the
// whole stage after a barrier; the ring kernel uses the per-wave regions of
// make_wave_loads instead). Per-thread constants: load l of wave wv covers
// stage pieces [(wv*NL + l)*64, +64): whole rows of tpi = 1024 / (hpu*RB) consecutive
// tokens of one plane (tpi divides ts and bs, so the 1 KiB a load covers never
// crosses a page). A wave's NL loads are consecutive pieces: with nw >= 2 they
// lie in one plane and span 32 / hpu tokens, so they touch at most two pages
// of the item (one when bs >= 32 / hpu); with nw = 1 (one page per item) the
// first half reads the K plane and the second half the V plane of that page.
// voff is the lane's byte offset from the start of its page, minus the item's
// offset inside the page (toff rows, when a page holds several items) and the
// head group's offset; both are added per item as scalars.
template <int KIND, int D>
struct LoadPlan {
  uint32_t voff[Geo<KIND, D>::NL];
  int vplane;     // bit l: load l reads the V plane (uniform)
  int second;     // bit l: load l reads the wave's second page (uniform)
  int pi0, pi1;   // item-relative index of the first and second page (uniform)
  bool one_base;  // every load reads the first page, all in one plane (uniform)
};

template <int KIND, int D>
__device__ __forceinline__ void make_load_plan(const AttnParams& p, LoadPlan<KIND, D>& lp) {
  using G_ = Geo<KIND, D>;
  const int lane = threadIdx.x & 63, wv = uni(threadIdx.x >> 6);
  const int plane_pieces = (p.ts * G_::CPR) << p.lhpu;
  const uint32_t tok_stride = (uint32_t)p.Hkv * G_::RB;
  // items start on a page boundary when ts >= bs and inside one page otherwise
  const bool paged = p.ts >= (1 << p.lbs);
  lp.vplane = 0;
  lp.second = 0;
  lp.pi0 = 0;
  lp.pi1 = 0;
#pragma unroll
  for (int l = 0; l < G_::NL; ++l) {
    const int cb = (wv * G_::NL + l) * 64;               // first piece of the load (uniform)
    const int plane = cb >= plane_pieces ? 1 : 0;
    const int ccb = cb - plane * plane_pieces;
    const int tau0 = (ccb / G_::CPR) >> p.lhpu;
    const int cc = ccb + lane;
    const int row = cc / G_::CPR, pos = cc % G_::CPR;
    const int tau = row >> p.lhpu, hl = row & ((1 << p.lhpu) - 1);
    const int j = pos ^ (tau & (G_::CPR - 1));
    const int pi = paged ? tau0 >> p.lbs : 0;
    const int slot = paged ? tau & ((1 << p.lbs) - 1) : tau;  // token row inside the page
    lp.voff[l] = (uint32_t)slot * tok_stride + (uint32_t)hl * G_::RB + 16u * j;
    lp.vplane |= plane << l;
    if (l == 0) lp.pi0 = pi;
    if (pi != lp.pi0) {
      lp.pi1 = pi;
      lp.second |= 1 << l;
    }
  }
  lp.one_base = lp.second == 0 && (lp.vplane == 0 || lp.vplane == (1 << G_::NL) - 1);
}

// The two pages a wave's loads of an item read, looked up one loop iteration
// before the loads are issued (scalar loads; the wait for them falls on the
// next iteration's issue, not on the compute in between). A page index past
// the sequence's last page is clamped to it: such a page only feeds masked
// tokens.
struct PageSet {
  uint32_t phys0, phys1;  // block ids are >= 0: zero-extended, no use right after the load
};

template <int KIND, int D, bool SPARSE = false>
__device__ __forceinline__ void load_pages(const AttnParams& p, const int32_t* __restrict__ table,
                                           const ItemPos& it, const LoadPlan<KIND, D>& lp,
                                           PageSet& pg) {
  if constexpr (SPARSE) {
    // an item is one plan entry (one page): every load of it reads that page
    const uint32_t phys = (uint32_t)p.sp_entries[2 * ((size_t)it.b * p.sp_cap + it.k)];
    pg.phys0 = phys;
    pg.phys1 = phys;
    return;
  }
  const int blk0 = (it.k << p.lts) >> p.lbs;
  const int last_blk = (it.L - 1) >> p.lbs;
  const int32_t* table_row = table + (size_t)it.b * p.max_blocks;
  pg.phys0 = (uint32_t)table_row[min(blk0 + lp.pi0, last_blk)];
  pg.phys1 = (uint32_t)table_row[min(blk0 + lp.pi1, last_blk)];
}

// Issue the workgroup-wide stage loads of one item into `slot`. Every thread issues exactly NL
// loads whether the item is live or not. Stage layout: K plane then V plane,
// each [TS tokens][HPU heads][CPR pieces]; piece j of row (tau, hl) is stored
// at position j ^ (tau & (CPR - 1)). Each load's address is a scalar page base
// plus the lane's constant offset; the page bases are formed once per item in
// 32 x 32 -> 64-bit products.
template <int KIND, int D>
__device__ __forceinline__ void issue_stage(const AttnParams& p, const ItemPos& it,
                                            const PageSet& pg, bool live,
                                            const LoadPlan<KIND, D>& lp, uint8_t* slot) {
  using G_ = Geo<KIND, D>;
  const int wv = uni(threadIdx.x >> 6);
  uint8_t* dst = slot + wv * G_::NL * 1024;
  if (live) {
    const uint32_t toff = (uint32_t)(it.k << p.lts) & ((1u << p.lbs) - 1u);  // 0 unless a page holds several items
    const uint32_t tok_stride = (uint32_t)p.Hkv * G_::RB;
    const uint32_t page_stride = tok_stride << p.lbs;
    const uint32_t item_off = toff * tok_stride + (((uint32_t)it.hg * G_::RB) << p.lhpu);
    uint64_t off0 = (uint64_t)pg.phys0 * page_stride + item_off;
    if (lp.one_base) {
      // the usual case: one page and one plane for all of the wave's loads
      const uint8_t* base = (lp.vplane ? p.v_cache : p.k_cache) + off0;
#pragma unroll
      for (int l = 0; l < G_::NL; ++l) dma16(base, lp.voff[l], dst + l * 1024);
    } else {
      // both products formed once (as uniform values): otherwise the compiler
      // selects the page id per load and redoes the multiply
      off0 = uni64(off0);
      const uint64_t off1 = uni64((uint64_t)pg.phys1 * page_stride + item_off);
#pragma unroll
      for (int l = 0; l < G_::NL; ++l) {
        const uint8_t* base = ((lp.vplane >> l) & 1) ? p.v_cache : p.k_cache;
        dma16(base + (((lp.second >> l) & 1) ? off1 : off0), lp.voff[l], dst + l * 1024);
      }
    }
  } else {
    // past the end of the range: the same number of loads, of 16 readable
    // bytes, into a slot nobody reads
    const uint8_t* sbase = reinterpret_cast<const uint8_t*>(p.q);
#pragma unroll
    for (int l = 0; l < G_::NL; ++l) dma16(sbase, 0u, dst + l * 1024);
  }
}

// ---------------------------------------------------------------------------
// Ring kernel loads, one region per wave. Wave (hl, st) computes head hl of
// the group for tokens [16 st, 16 st + 16) of an item; it also loads exactly
// those K and V rows into a region of its own, [K: 16 rows][V: 16 rows] of RB
// bytes, with the 16-byte pieces of row r stored at position j ^ (r & (CPR-1)).
// No wave reads another wave's region, so a wave waits for its own loads only
// and the ring needs no barrier per stage. The 16 tokens never cross a page
// (bs >= 16), so every item costs a wave one block-table lookup.
template <int KIND, int D>
struct WaveLoads {
  uint32_t voff[Geo<KIND, D>::NL];  // loads [0, NL/2) read K rows, the rest V rows
  int pi;                           // item-relative page of the wave's tokens (uniform)
};

template <int KIND, int D>
__device__ __forceinline__ void make_wave_loads(const AttnParams& p, int st, int hl,
                                                WaveLoads<KIND, D>& wl) {
  using G_ = Geo<KIND, D>;
  constexpr int CPR = G_::CPR, RB = G_::RB, NL = G_::NL, HALF = NL / 2, TPR = 1024 / RB;
  static_assert(NL % 2 == 0 && 16 % TPR == 0 && HALF * TPR == 16, "per-wave load geometry");
  const int lane = threadIdx.x & 63;
  const uint32_t tok_stride = (uint32_t)p.Hkv * RB;
  const bool paged = p.ts >= (1 << p.lbs);  // items start on a page boundary
  const int t0 = 16 * st;
  wl.pi = paged ? t0 >> p.lbs : 0;
  const int slot0 = paged ? t0 & ((1 << p.lbs) - 1) : t0;
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const int r = (l % HALF) * TPR + lane / CPR, pos = lane % CPR;
    const int j = pos ^ (r & (CPR - 1));
    wl.voff[l] = (uint32_t)(slot0 + r) * tok_stride + (uint32_t)hl * RB + 16u * j;
  }
}

template <int KIND, int D, bool SPARSE = false>
__device__ __forceinline__ void load_page_w(const AttnParams& p, const int32_t* __restrict__ table,
                                            const ItemPos& it, const WaveLoads<KIND, D>& wl,
                                            PageSet& pg) {
  if constexpr (SPARSE) {
    pg.phys0 = (uint32_t)p.sp_entries[2 * ((size_t)it.b * p.sp_cap + it.k)];
  } else {
    const int blk0 = (it.k << p.lts) >> p.lbs;
    const int last_blk = (it.L - 1) >> p.lbs;
    pg.phys0 = (uint32_t)table[(size_t)it.b * p.max_blocks + min(blk0 + wl.pi, last_blk)];
  }
}

// Issue a wave's NL loads of one item into its region `dst` (the same number
// whether the item is live or not).
template <int KIND, int D>
__device__ __forceinline__ void issue_w(const AttnParams& p, const ItemPos& it, const PageSet& pg,
                                        bool live, const WaveLoads<KIND, D>& wl, uint8_t* dst) {
  using G_ = Geo<KIND, D>;
  constexpr int NL = G_::NL;
  if (live) {
    const uint32_t toff = (uint32_t)(it.k << p.lts) & ((1u << p.lbs) - 1u);  // 0 unless a page holds several items
    const uint32_t tok_stride = (uint32_t)p.Hkv * G_::RB;
    const uint64_t off = (uint64_t)pg.phys0 * (tok_stride << p.lbs) + toff * tok_stride +
                         (((uint32_t)it.hg * G_::RB) << p.lhpu);
    const uint8_t* kb = p.k_cache + off;
    const uint8_t* vb = p.v_cache + off;
#pragma unroll
    for (int l = 0; l < NL; ++l) dma16(l < NL / 2 ? kb : vb, wl.voff[l], dst + l * 1024);
  } else {
    const uint8_t* sbase = reinterpret_cast<const uint8_t*>(p.q);
#pragma unroll
    for (int l = 0; l < NL; ++l) dma16(sbase, 0u, dst + l * 1024);
  }
}

// Softmax state and Q' operands of one wave.
template <int KIND, int D, int RT, int QF>
struct WaveState {
  h8 qa[RT][Geo<KIND, D>::KS];
  h8 qb[RT][QF == kQSplit ? Geo<KIND, D>::KS : 1];
  f4 o[RT][Geo<KIND, D>::DV];
  float m_run[RT];
  f4 l_acc[RT];  // row sums of P, accumulated by the matrix cores (all 4 lanes of a row equal)
  int lim[RT];  // query row 16*rt+n sees tokens t <= lim
};

// Eight channels of a q row as fp32: fp16 values, or bf16 bits widened (a
// bf16 value is the upper half of an fp32).
__device__ __forceinline__ void load_q8(const uint16_t* src, bool bf16, bool valid, float* x) {
  u4 raw = {0u, 0u, 0u, 0u};
  if (valid) raw = *reinterpret_cast<const u4*>(src);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (bf16) {
      x[2 * k] = __uint_as_float(raw[k] << 16);
      x[2 * k + 1] = __uint_as_float(raw[k] & 0xFFFF0000u);
    } else {
      const h2 v = as_h2(raw[k]);
      x[2 * k] = (float)v[0];
      x[2 * k + 1] = (float)v[1];
    }
  }
}

// Row of the run's block that lane column n of row tile rt holds.
template <int QF>
__device__ __forceinline__ int lane_row(int rt, int n) {
  return qf_pack(QF) ? (n & 7) : 16 * rt + n;
}

// Load Q' of (sequence b, row block rb, KV head hk) and reset the softmax
// state. Local row lane_row(rt, n) is query row rb * rpb + that row.
template <int KIND, int D, int RT, int QF>
__device__ __forceinline__ void start_run(const AttnParams& p, int b, int rb, int hk, int L,
                                          float inv_m, float sgn,
                                          WaveState<KIND, D, RT, QF>& w) {
  using G_ = Geo<KIND, D>;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rl = lane_row<QF>(rt, n), r = rb * p.rpb + rl;
    const bool rv = rl < p.rpb && r < p.R;
    const int i = r / p.G, hg = r % p.G;
    const uint16_t* qrow = p.q + (((size_t)b * p.next_n + i) * p.Hq + hk * p.G + hg) * D;
#pragma unroll
    for (int ks = 0; ks < G_::KS; ++ks) {
      const int j = ks / G_::KPC, u = ks % G_::KPC;
      const int d0 = (g + 4 * j) * G_::EPC + 8 * u;
      float xv[8];
      load_q8(qrow + d0, p.q_bf16, rv, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + run_elem<KIND>(e);
        const float x = xv[run_elem<KIND>(e)];
        if constexpr (qf_fold(QF)) {
          const float xf = x * (p.k_scale[hk * D + d] * inv_m) * sgn;
          const _Float16 hi = (_Float16)xf;
          const _Float16 lo = (_Float16)(xf - (float)hi);
          if constexpr (QF == kQPacked) {
            w.qa[rt][ks][e] = n < 8 ? hi : lo;
          } else {
            w.qa[rt][ks][e] = hi;
            w.qb[rt][ks][e] = lo;
          }
        } else {
          w.qa[rt][ks][e] = (_Float16)(x * sgn);
        }
      }
    }
    w.m_run[rt] = -INFINITY;
    w.l_acc[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < G_::DV; ++q) w.o[rt][q] = f4{0.f, 0.f, 0.f, 0.f};
    w.lim[rt] = p.causal ? (L - p.next_n + i) : 0x7fffffff;
  }
}

// LDS byte offsets (within a wave's region of a stage) of the pieces a lane
// reads in compute_tile: K pieces g + 4j of the sub-tile's token n, and V
// bytes [n*VB, n*VB + VB) of its tokens 4g + e.
template <int KIND, int D>
struct TileOffs {
  static constexpr int VP = Geo<KIND, D>::VB >= 16 ? Geo<KIND, D>::VB / 16 : 1;
  int k[Geo<KIND, D>::NJ];
  int v[4][VP];
};

// Offsets inside a wave's own region (see make_wave_loads): K rows 0..15,
// then V rows 0..15, RB bytes each.
template <int KIND, int D>
__device__ __forceinline__ void make_tile_offs_w(TileOffs<KIND, D>& to) {
  using G_ = Geo<KIND, D>;
  constexpr int CPR = G_::CPR, RB = G_::RB, VB = G_::VB;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < G_::NJ; ++j) to.k[j] = n * RB + 16 * ((g + 4 * j) ^ (n & (CPR - 1)));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tau = 4 * g + e;
    const int row = 16 * RB + tau * RB;
    const int byte = n * VB;
#pragma unroll
    for (int pp = 0; pp < TileOffs<KIND, D>::VP; ++pp)
      to.v[e][pp] = row + 16 * ((byte / 16 + pp) ^ (tau & (CPR - 1))) + (VB < 16 ? byte % 16 : 0);
  }
}

// max over the four 16-lane rows of the wave (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Codes of the same dword of two tokens, regrouped so that each fp16 pair the
// kind's decode produces is (token a, token b) of one channel, in natural
// channel order: the first dword gives channels [0, P) of the dword's run, the
// second [P, 2P) (P = pairs per dword). 8-bit codes interleave bytes; 4-bit and
// 16-bit codes put the low halves, then the high halves, of the two tokens
// side by side (an INT4 decode pairs nibbles k and k + 4).
template <int KIND>
__device__ __forceinline__ void pair_tokens(uint32_t xa, uint32_t xb, uint32_t& y0, uint32_t& y1) {
  if constexpr (Kv<KIND>::kBits == 8) {
    y0 = __builtin_amdgcn_perm(xb, xa, 0x05010400u);
    y1 = __builtin_amdgcn_perm(xb, xa, 0x07030602u);
  } else {
    y0 = __builtin_amdgcn_perm(xb, xa, 0x05040100u);
    y1 = __builtin_amdgcn_perm(xb, xa, 0x07060302u);
  }
}

// The two fp16 parts of a softmax weight: hi = fp16(x), lo = fp16(x - hi)
// (x - hi is exact in fp32).
__device__ __forceinline__ _Float16 p_lo(float x, _Float16 hi) { return (_Float16)(x - (float)hi); }

// Softmax step of one row tile: new running max, rescale factor, P as the B
// operand of the P V product (PACK: the k = 16 form, lanes n < 8 the high
// parts and n >= 8 the remainders, in pb[0..3]; otherwise the k = 32 form,
// high parts in pb[0..3] and remainders in pb[4..7]). MASK = false when every
// query row sees all 16 tokens (none past the end or past a row's causal
// limit): no selects then.
template <bool MASK, bool PACK>
__device__ __forceinline__ void tile_softmax(const f4 s, uint32_t okbits, float c2, float& m_run,
                                             float& alpha, bool& rescale, h8& pb) {
  bool okv[4];
  float mx;
  if constexpr (MASK) {
    mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      okv[e] = (okbits >> e) & 1u;
      mx = okv[e] ? fmaxf(mx, s[e]) : mx;
    }
  } else {
    mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  }
  mx = rows_max(mx);
  const float m_old = m_run;
  const float m_new = fmaxf(m_old, mx);
  // the state needs rescaling only when a row that has seen tokens gets a
  // larger max; a row that has seen nothing holds zeros
  alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_old - m_new) * c2);
  rescale |= m_old != m_new && m_old != -INFINITY;
  // exponent s * c2 - (m * c2 - kPScale) as one fma (a row that saw only
  // masked tokens keeps m = -inf; its p are selected to 0)
  const float mc = m_new == -INFINITY ? 0.f : m_new * c2 - kPScale;
  float pf[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pf[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c2, -mc));
    if constexpr (MASK) pf[e] = okv[e] ? pf[e] : 0.f;
  }
  if constexpr (PACK) {
    const bool hi_lane = (threadIdx.x & 15) < 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 hi = (_Float16)pf[e];
      pb[e] = hi_lane ? hi : p_lo(pf[e], hi);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 hi = (_Float16)pf[e];
      pb[e] = hi;
      pb[4 + e] = p_lo(pf[e], hi);
    }
  }
  m_run = m_new;
}

// One 16-token sub-tile (tokens t0 .. t0 + 15) of the wave's head from a ring
// slot. full: every query row sees all 16 tokens (wave-uniform), so the
// softmax and the V codes need no masking. SPARSE: token 4g + e of the
// sub-tile is valid for the lane's row when bit tin + 4g + e of rmask[rt] is
// set (tin = the sub-tile's first token in its page), and its V codes are
// kept when that bit is set in umask (some row selected it).
template <int KIND, int D, int RT, int QF, bool SPARSE = false>
__device__ __forceinline__ void compute_tile(const uint8_t* slot, const TileOffs<KIND, D>& to,
                                             int t0, int L, bool full, float c2,
                                             WaveState<KIND, D, RT, QF>& w,
                                             const uint32_t* rmask = nullptr, uint32_t umask = 0,
                                             int tin = 0) {
  using G_ = Geo<KIND, D>;
  constexpr int KS = G_::KS, NJ = G_::NJ, KPC = G_::KPC, EPC = G_::EPC, DV = G_::DV;
  constexpr int VDW = G_::VDW, VB = G_::VB;
  constexpr int P = Kv<KIND>::kPairsPerDword;
  constexpr bool PACK = qf_pack(QF);
  static_assert(VDW * 2 * P == DV, "V channels per lane");
  static_assert(!PACK || RT == 1, "packed rows fill one row tile");
  const int lane = threadIdx.x & 63, g = lane >> 4;

  // ---- K operand: lane (n, g) holds token n, pieces g + 4j ----
  h8 kop[KS];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const u4 raw = *reinterpret_cast<const u4*>(slot + to.k[j]);
    _Float16 hv[EPC];
    uint32_t wd[4] = {raw[0], raw[1], raw[2], raw[3]};
    decode_run<KIND, 4>(wd, hv);
#pragma unroll
    for (int u = 0; u < KPC; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) kop[j * KPC + u][e] = hv[8 * u + e];
  }
  // ---- V codes: lane (n, g) holds tokens 4g + e, row bytes [n*VB, n*VB + VB) ----
  uint32_t vraw[4][VDW];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (VB >= 16) {
#pragma unroll
      for (int pp = 0; pp < VB / 16; ++pp) {
        const u4 x = *reinterpret_cast<const u4*>(slot + to.v[e][pp]);
#pragma unroll
        for (int k = 0; k < 4; ++k) vraw[e][4 * pp + k] = x[k];
      }
    } else if constexpr (VDW == 2) {
      const u2 x = *reinterpret_cast<const u2*>(slot + to.v[e][0]);
      vraw[e][0] = x[0];
      vraw[e][1] = x[1];
    } else {
      vraw[e][0] = *reinterpret_cast<const uint32_t*>(slot + to.v[e][0]);
    }
  }
  if (__builtin_expect(!full, 0)) {
    // tokens past the end (or selected by no row): zero their V codes by
    // select, so no 0 * NaN can reach O [NULLPAD, Fix]
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool ok;
      if constexpr (SPARSE)
        ok = (umask >> (tin + 4 * g + e)) & 1u;
      else
        ok = t0 + 4 * g + e < L;
#pragma unroll
      for (int k = 0; k < VDW; ++k) vraw[e][k] = ok ? vraw[e][k] : 0u;
    }
  }

  f4 sacc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], w.qa[rt][ks], acc, 0, 0, 0);
      if constexpr (QF == kQSplit)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], w.qb[rt][ks], acc, 0, 0, 0);
    }
    if constexpr (QF == kQPacked) {
      // column n + high part of its row, from column (n + 8) mod 16 (row_ror:8);
      // both halves of the row end up with the same sum
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] += __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(acc[e]), 0x128, 0xF, 0xF, false));
    }
    sacc[rt] = acc;
  }

  // ---- online softmax (query row = lane column n) ----
  h8 pb[RT];
  bool rescale = false;
  float alpha[RT];
  if (full) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      tile_softmax<false, PACK>(sacc[rt], 0xFu, c2, w.m_run[rt], alpha[rt], rescale, pb[rt]);
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t okbits = 0;
      if constexpr (SPARSE) {
        okbits = (rmask[rt] >> (tin + 4 * g)) & 0xFu;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = t0 + 4 * g + e;
          okbits |= (uint32_t)(t < L && t <= w.lim[rt]) << e;
        }
      }
      tile_softmax<true, PACK>(sacc[rt], okbits, c2, w.m_run[rt], alpha[rt], rescale, pb[rt]);
    }
  }
  if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int q = 0; q < DV; ++q) w.o[rt][q] *= alpha[rt];
      w.l_acc[rt] *= alpha[rt];
    }
  }

  // ---- O^T += V^T P^T: the A operand of channel q is (tokens 4g .. 4g+3) of
  // that channel, built straight from decodes of token-paired codes (and
  // repeated for the remainder slots of the k = 32 form) ----
#pragma unroll
  for (int k = 0; k < VDW; ++k) {
    // dword k of the lane's run: channels [2Pk, 2Pk + 2P), decoded and used at once
    uint32_t y[4];
    pair_tokens<KIND>(vraw[0][k], vraw[1][k], y[0], y[1]);
    pair_tokens<KIND>(vraw[2][k], vraw[3][k], y[2], y[3]);
    h2 pr[4][P];
#pragma unroll
    for (int i = 0; i < 4; ++i) Kv<KIND>::decode(y[i], pr[i]);
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) {
      const h2 a = pr[i < P ? 0 : 1][i % P], b = pr[i < P ? 2 : 3][i % P];
      const int q = 2 * P * k + i;
      if constexpr (PACK) {
        const h4 vop = {a[0], a[1], b[0], b[1]};
        const h4 pb4 = {pb[0][0], pb[0][1], pb[0][2], pb[0][3]};
        w.o[0][q] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, pb4, w.o[0][q], 0, 0, 0);
      } else {
        const h8 vop = {a[0], a[1], b[0], b[1], a[0], a[1], b[0], b[1]};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          w.o[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pb[rt], w.o[rt][q], 0, 0, 0);
      }
    }
  }
  // row sums of P on the matrix cores: every lane gets its row's sum
  if constexpr (PACK) {
    const h4 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
    const h4 pb4 = {pb[0][0], pb[0][1], pb[0][2], pb[0][3]};
    w.l_acc[0] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pb4, w.l_acc[0], 0, 0, 0);
  } else {
    const h8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                     (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      w.l_acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[rt], w.l_acc[rt], 0, 0, 0);
  }
}

// Exchange of one row tile of a wave's softmax state through LDS, in the MFMA
// register layout (lane-major), so the receiving wave of the same head
// combines element-wise: o as [q][lane] f4, then m and l as [lane] floats
// (D / 16 KiB + 512 bytes). One row tile at a time keeps the buffer small
// enough for every head_dim and the live registers few.
template <int KIND, int D, int RT, int QF>
__device__ __forceinline__ void xch_put(const WaveState<KIND, D, RT, QF>& w, int rt, float* xbuf) {
  constexpr int DV = Geo<KIND, D>::DV;
  const int lane = threadIdx.x & 63;
  f4* xo = reinterpret_cast<f4*>(xbuf);
#pragma unroll
  for (int q = 0; q < DV; ++q) xo[q * 64 + lane] = w.o[rt][q];
  xbuf[DV * 256 + lane] = w.m_run[rt];
  xbuf[DV * 256 + 64 + lane] = w.l_acc[rt][0];
}

// Combine row tile rt of the state in xbuf into w (w first, then xbuf: a
// fixed order).
template <int KIND, int D, int RT, int QF>
__device__ __forceinline__ void xch_merge(WaveState<KIND, D, RT, QF>& w, int rt, const float* xbuf,
                                          float c2) {
  constexpr int DV = Geo<KIND, D>::DV;
  const int lane = threadIdx.x & 63;
  const f4* xo = reinterpret_cast<const f4*>(xbuf);
  {
    const float mb = xbuf[DV * 256 + lane];
    const float lb = xbuf[DV * 256 + 64 + lane];
    const float ma = w.m_run[rt];
    const float mn = fmaxf(ma, mb);
    const float a = ma == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ma - mn) * c2);
    const float bw = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mb - mn) * c2);
    const float l = w.l_acc[rt][0] * a + lb * bw;
    w.l_acc[rt] = f4{l, l, l, l};
    w.m_run[rt] = mn;
#pragma unroll
    for (int q = 0; q < DV; ++q) {
      w.o[rt][q] = w.o[rt][q] * a + xo[q * 64 + lane] * bw;
      __builtin_amdgcn_sched_barrier(0);  // keep one f4 in flight: register pressure
    }
  }
}

// Barrier over the workgroup that leaves the ring loads in flight: LDS writes
// are waited for, vector memory is not.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Partial index of (run r, workgroup w, head-in-group hl); run
// r = (b * nrb + rb) * hgroups + hg. Slot r + w is unique: a later workgroup only reaches
// later runs, so (r, w) != (r', w') with r + w == r' + w' cannot both occur.
__device__ __forceinline__ size_t part_index(const AttnParams& p, int r, int w, int hl) {
  return (size_t)(r + w) * p.hpu + hl;
}

// Adds column (n + 8) mod 16 of a packed state to column n (row_ror:8): the
// remainder half of P's products joins the high half.
__device__ __forceinline__ float add_ror8(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF,
                                                        false));
}

// Write the wave's state as a partial. A packed state's halves are added
// first, in place (the state is reset by the next start_run).
template <int KIND, int D, int RT, int QF>
__device__ __forceinline__ void write_partial(const AttnParams& p, size_t u, float c2,
                                              WaveState<KIND, D, RT, QF>& w, int row0 = 0) {
  constexpr int DV = Geo<KIND, D>::DV;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if constexpr (qf_pack(QF)) {
      // lanes n < 8 hold the products of P's high parts, n + 8 the remainders
      w.l_acc[rt][0] = add_ror8(w.l_acc[rt][0]);
#pragma unroll
      for (int q = 0; q < DV; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) w.o[rt][q][e] = add_ror8(w.o[rt][q][e]);
    }
    // row of the run's block; packed states write from lanes n < 8 only
    const int r = row0 + 16 * rt + n;
    if (r < p.rpb && (!qf_pack(QF) || n < 8)) {
      if (g == 0) p.ws_ml[u * p.rpb + r] = f4{w.m_run[rt], w.l_acc[rt][0], c2, 0.f};
      float* orow = p.ws_o + (u * p.rpb + r) * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float tmp[DV];
#pragma unroll
        for (int q = 0; q < DV; ++q) tmp[q] = w.o[rt][q][e];
#pragma unroll
        for (int k = 0; k < DV; k += 4)
          *reinterpret_cast<f4*>(orow + DV * (4 * g + e) + k) =
              f4{tmp[k], tmp[k + 1], tmp[k + 2], tmp[k + 3]};
      }
    }
  }
}

// Row masks of one plan entry (sparse mode): next_n words, scalar loads.
constexpr int kSparseRows = 4;  // next_n limit of the sparse mode
constexpr int kPlanWords = 512; // page bitmap words of the union planner (16384 pages)

__device__ __forceinline__ void load_row_masks(const AttnParams& p,
                                               const uint32_t* __restrict__ masks,
                                               const ItemPos& it, uint32_t* m) {
  const size_t base = ((size_t)it.b * p.sp_cap + it.k) * p.next_n;
#pragma unroll
  for (int i = 0; i < kSparseRows; ++i) m[i] = i < p.next_n ? masks[base + i] : 0u;
}

// This workgroup's item range, computed by one wave (see the cost line in
// the kernel below); lane 0 leaves {count, b, hg, k, L, rb} of the first item
// in xi[0..5] and the range's first global item index in xi[6]. Workgroup 0 also publishes every sequence's first slot and the
// slot total for the merge kernel.
__device__ __forceinline__ void range_scan(const AttnParams& p, const int32_t* __restrict__ lens,
                                           int* xi) {
  const int lane = threadIdx.x & 63;
  int ccarry = 0;
  const int len_first = lane < p.B ? lens[lane] : 0;  // kept for the second pass
  for (int base = 0; base < p.B; base += 64) {
    const int b = base + lane;
    int cost, items;
    seq_cost(p, base == 0 ? len_first : (b < p.B ? lens[b] : 0), cost, items);
    const int incl = wave_incl_scan(cost);
    if (blockIdx.x == 0 && b < p.B) p.ws_seq[b] = ccarry + incl - cost;
    ccarry += lane_val(incl, 63);
  }
  if (blockIdx.x == 0 && lane == 0) p.ws_seq[p.B] = ccarry;
  const int qc = max(1, (ccarry + p.nwg - 1) / p.nwg);
  const int ta = (int)blockIdx.x * qc, tz = ta + qc;  // this workgroup's slots
  // first item at or after slot ta (and tz): sequence, row block, head
  // group, stage, index
  int fb = -1, fL = 0, frb = 0, fhg = 0, fk = 0, ia = -1, iz = -1;
  int c0 = 0, n0 = 0;
  for (int base = 0; base < p.B; base += 64) {
    const int b = base + lane;
    const int len = base == 0 ? len_first : (b < p.B ? lens[b] : 0);
    int cost, items;
    seq_cost(p, len, cost, items);
    const int ic = wave_incl_scan(cost), ii = wave_incl_scan(items);
    const int ec = c0 + ic - cost, ei = n0 + ii - items;
    // the first non-empty sequence whose slots end past t holds slot t
    const uint64_t hit_a = ia >= 0 ? 0 : __builtin_amdgcn_ballot_w64(cost > 0 && ec + cost > ta);
    const uint64_t hit_z = __builtin_amdgcn_ballot_w64(cost > 0 && ec + cost > tz);
    if (hit_a) {
      const int f = __builtin_ctzll(hit_a);
      fb = base + f;
      fL = lane_val(len, f);
      ia = lane_val(ei, f) + locate_slot(p, fL, ta - lane_val(ec, f), frb, fhg, fk);
    }
    if (hit_z) {
      const int f = __builtin_ctzll(hit_z);
      int zrb, zhg, zk;
      iz = lane_val(ei, f) + locate_slot(p, lane_val(len, f), tz - lane_val(ec, f), zrb, zhg, zk);
      break;
    }
    c0 += lane_val(ic, 63);
    n0 += lane_val(ii, 63);
  }
  // slots past the last sequence: the range ends at the item total
  if (ia < 0) ia = n0;
  if (iz < 0) iz = n0;
  if (lane == 0) {
    xi[0] = iz - ia;
    xi[1] = fb;
    xi[2] = fhg;
    xi[3] = fk;
    xi[4] = fL;
    xi[5] = frb;
    xi[6] = ia;  // global index of the range's first item
  }
}

// Ring kernel modes: dense (one row block), selection-driven sparse, and dense
// with several query row blocks per sequence.
enum RingMode { kModeDense = 0, kModeSparse = 1, kModeRows = 2 };

// MODE kModeSparse: table holds the union plan entries ({physical, logical}
// per page), lens the per-sequence entry count times block_size, masks the row
// masks. kModeRows: query rows come in p.nrb blocks of p.rpb rows.
template <int KIND, int D, int RT, int QF, int NWB, int MODE>
__global__ __launch_bounds__(64 * NWB) void attn_ring_kernel(
    AttnParams p, const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
    const uint32_t* __restrict__ masks) {
  constexpr bool SPARSE = MODE == kModeSparse;
  using G_ = Geo<KIND, D>;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * kStageMax];
  const int lane = threadIdx.x & 63, wv = uni(threadIdx.x >> 6);  // wave-uniform
  const int hl = wv & (p.hpu - 1), st = wv >> p.lhpu;
  const int stage_bytes = (2 * p.ts * G_::RB) << p.lhpu;
  __shared__ __attribute__((aligned(16))) float xbuf[kXchBytes / 4];
  int* xi = reinterpret_cast<int*>(xbuf);
  // one row block outside kModeRows: the block logic folds away
  if constexpr (MODE != kModeRows) {
    p.nrb = 1;
    p.rpb = p.R;
  }
  // ---- this workgroup's item range. Items are placed on a cost line where
  // each (sequence, row block, head group) run first takes run_cost empty slots (the
  // pipeline drain at a run start) and then one slot per item; workgroup w
  // takes the items whose slots fall in [w*Qc, (w+1)*Qc). One wave scans the
  // sequence lengths; workgroup 0 also publishes every sequence's first slot
  // and the total for the merge kernel ----
  if (wv == 0) range_scan(p, lens, xi);
  // the per-tensor K scale: its pointer is a scalar load of its own, so it is
  // read after the scan's length load has gone out
  const float ks_tensor =
      (!qf_fold(QF) && p.k_scale_mode == PA_SCALE_PER_TENSOR) ? p.k_scale[0] : 1.0f;
  __syncthreads();
  // workgroup-uniform (read back from LDS, so say so to the compiler)
  const int nitems = uni(xi[0]);
  if (nitems <= 0) return;
  ItemPos cp;
  cp.b = uni(xi[1]);
  cp.L = uni(xi[4]);
  cp.rb = MODE != kModeRows ? 0 : uni(xi[5]);
  cp.nst = run_stages(p, cp.L, cp.rb);
  cp.hg = uni(xi[2]);
  cp.k = uni(xi[3]);

  WaveLoads<KIND, D> wl;
  make_wave_loads<KIND, D>(p, st, hl, wl);
  TileOffs<KIND, D> to;
  make_tile_offs_w<KIND, D>(to);
  // this wave's region of every ring stage
  uint8_t* const myring = ring + wv * (32 * G_::RB);

  WaveState<KIND, D, RT, QF> w;

  // ---- ring prologue: kStages - 1 items in flight; the block-table loads of
  // all of them (and of the next one) are issued before any is waited for ----
  ItemPos pos[kStages];
  pos[0] = cp;
#pragma unroll
  for (int j = 1; j < kStages; ++j) {
    pos[j] = pos[j - 1];
    if (j - 1 < nitems) item_next(p, lens, pos[j]);
  }
  // Unconditional lookups (an item past the range looks up the range's first
  // item instead, which is always valid) let every table load of the
  // prologue be issued before the first wait.
  PageSet pgs[kStages - 1];
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) {
    const bool in = j < nitems;
    ItemPos q;
    q.b = in ? pos[j].b : pos[0].b;
    q.L = in ? pos[j].L : pos[0].L;
    q.nst = in ? pos[j].nst : pos[0].nst;
    q.hg = in ? pos[j].hg : pos[0].hg;
    q.k = in ? pos[j].k : pos[0].k;
    q.rb = in ? pos[j].rb : pos[0].rb;
    load_page_w<KIND, D, SPARSE>(p, table, q, wl, pgs[j]);
  }
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    issue_w<KIND, D>(p, pos[j], pgs[j], j < nitems, wl, myring + j * stage_bytes);
  ItemPos ld = pos[kStages - 1];
  PageSet pg;
  if (kStages - 1 < nitems) load_page_w<KIND, D, SPARSE>(p, table, ld, wl, pg);

  // ---- scale constants, after the ring's first loads are on their way:
  // fold normalizer for PER_CHANNEL K [FOLD, Approach], max|k_scale| with 8
  // loads in flight per lane ----
  float qk, inv_m = 0.f;
  if constexpr (qf_fold(QF)) {
    float mx = 0.f;
    const int nks = p.Hkv * D;
    for (int i0 = 0; i0 < nks; i0 += 512) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + 64 * u + lane;
        v[u] = i < nks ? p.k_scale[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) mx = fmaxf(mx, fabsf(v[u]));
    }
    mx = wave_max(mx);
    inv_m = mx > 0.f ? 1.0f / mx : 0.f;
    qk = p.softmax_scale * mx;
  } else {
    qk = p.softmax_scale * ks_tensor;
  }
  const float sgn = qk < 0.f ? -1.f : 1.f;
  const float c2 = fabsf(qk) * kLog2e;

  // Q' of the first run: its loads follow the ring's first stages, so the
  // ring does not wait for them (the conversion waits for both; the first
  // compute needs the first stage anyway)
  start_run<KIND, D, RT, QF>(p, cp.b, cp.rb, cp.hg * p.hpu + hl, cp.L, inv_m, sgn, w);
  // SPARSE: row masks of the item being computed (mc) and of the next (mn),
  // loaded one iteration ahead; mp is the position of mn
  uint32_t mc[kSparseRows] = {0u, 0u, 0u, 0u}, mn[kSparseRows] = {0u, 0u, 0u, 0u};
  ItemPos mp = pos[1];
  if constexpr (SPARSE) {
    load_row_masks(p, masks, cp, mc);
    if (1 < nitems) load_row_masks(p, masks, mp, mn);
  }

  for (int j = 0; j < nitems; ++j) {
    // this wave's loads of item j have landed (its region is its own: no
    // barrier), and it is done with item j - 1, whose slot the next loads reuse
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kStages - 2) * G_::NL) : "memory");
    const int jn = j + kStages - 1;
    const bool live_n = jn < nitems;
    issue_w<KIND, D>(p, ld, pg, live_n, wl, myring + (jn % kStages) * stage_bytes);
    if (live_n) item_next(p, lens, ld);
    const int t0 = (cp.k << p.lts) + 16 * st;
    if constexpr (SPARSE) {
      // the lane's query row r = 16 rt + n reads the mask of step i = r / G
      uint32_t rm[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = lane_row<QF>(rt, lane & 15);
        const int i = r / p.G;
        uint32_t m = 0u;
#pragma unroll
        for (int k = 0; k < kSparseRows; ++k) m = i == k ? mc[k] : m;
        rm[rt] = r < p.rpb ? m : 0u;  // one row block in this mode
      }
      // this sub-tile's tokens: skipped when no row selected any, unmasked
      // when every row selected all (wave-uniform: the masks are scalar)
      uint32_t any = 0u, all = ~0u;
#pragma unroll
      for (int k = 0; k < kSparseRows; ++k) {
        any |= mc[k];
        all &= k < p.next_n ? mc[k] : ~0u;
      }
      const uint32_t sub_any = (any >> (16 * st)) & 0xFFFFu;
      const uint32_t sub_all = (all >> (16 * st)) & 0xFFFFu;
      if (sub_any != 0u)
        compute_tile<KIND, D, RT, QF, true>(myring + (j % kStages) * stage_bytes, to, t0, cp.L,
                                              sub_all == 0xFFFFu, c2, w, rm, any, 16 * st);
    } else if (t0 < run_len(p, cp.L, cp.rb)) {
      // full: the block's first row (step first_step) sees all 16 tokens
      compute_tile<KIND, D, RT, QF>(
          myring + (j % kStages) * stage_bytes, to, t0, cp.L,
          t0 + 16 <= cp.L - (p.causal ? p.next_n - 1 - first_step(p, cp.rb) : 0), c2, w);
    }
    // end of a (sequence, head group) run inside this range: write the partial
    const int b = cp.b, hg = cp.hg, rb = cp.rb;
    item_next(p, lens, cp);
    if (j + 1 == nitems || cp.b != b || cp.hg != hg || cp.rb != rb) {
      const int run = (b * p.nrb + rb) * p.hgroups + hg;
      if (p.nsub > 1) {
        // fold sub-tiles 1 .. nsub-1 of each head into sub-tile 0, in order,
        // one row tile at a time
        for (int h = 0; h < p.hpu; ++h)
          for (int s2 = 1; s2 < p.nsub; ++s2)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              if (hl == h && st == s2) xch_put<KIND, D, RT, QF>(w, rt, xbuf);
              lds_barrier();
              if (hl == h && st == 0) xch_merge<KIND, D, RT, QF>(w, rt, xbuf, c2);
              lds_barrier();
            }
      }
      if (st == 0)
        write_partial<KIND, D, RT, QF>(p, part_index(p, run, blockIdx.x, hl), c2, w);
      if (j + 1 < nitems)
        start_run<KIND, D, RT, QF>(p, cp.b, cp.rb, cp.hg * p.hpu + hl, cp.L, inv_m, sgn, w);
    }
    // pages of the item the next iteration issues
    if (jn + 1 < nitems) load_page_w<KIND, D, SPARSE>(p, table, ld, wl, pg);
    if constexpr (SPARSE) {
#pragma unroll
      for (int k = 0; k < kSparseRows; ++k) mc[k] = mn[k];
      if (j + 2 < nitems) {
        item_next(p, lens, mp);
        load_row_masks(p, masks, mp, mn);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Prefill layout: hundreds of query rows per KV head
// ---------------------------------------------------------------------------
// In the ring kernel's row-block mode every block of 32 rows decodes the same
// K and V again. Here the 8 waves of a workgroup are 8 row blocks (a group of
// 256 rows) of one KV head: a stage holds 128 tokens of that head, the waves
// decode it once together into fp16 in LDS, and each wave then runs all 8
// sub-tiles of 16 tokens for its own 32 rows from the decoded copy. Runs are
// (sequence, row group, KV head) and items are 128-token stages: the cost
// line, item order, partials and merge are those of the ring kernel with one
// head per group (hpu 1), 128-token items and 256-row blocks.
constexpr int kPfWaves = 8;
constexpr int kPfTokens = 128;  // tokens per stage
constexpr int kPfStages = 3;    // ring stages (two in flight while one is computed)
constexpr int kPfMinRows = 128; // query rows per KV head from which the prefill layout is used

template <int KIND, int D>
struct PfGeo {
  using G_ = Geo<KIND, D>;
  static constexpr int PPR = D / 8;                    // 16-byte pieces of a decoded K row
  static constexpr int SLOTS = kPfTokens / 4;          // 8-byte token quads of a decoded V row
  static constexpr int STAGE = 2 * kPfTokens * G_::RB;  // K and V codes of one stage
  static constexpr int KDEC = kPfTokens * D * 2;        // fp16 K, [token][channel]
  static constexpr int VDEC = D * kPfTokens * 2;        // fp16 V, [channel][token]
  static constexpr int BPE = G_::BITS;                  // code bytes of 8 channels of a token
  static constexpr int LDS = kPfStages * STAGE + KDEC + VDEC;
  static constexpr bool OK = D <= 128 && STAGE <= kStageMax && LDS <= 160 * 1024;
};

// Decode one landed stage into kdec / vdec. Block (tb, cb) = tokens 4 tb ..
// 4 tb + 3, channels 8 cb .. 8 cb + 7 of both planes. In the ring slot the
// piece j of token tau sits at j ^ (tau & (CPR - 1)); in kdec piece c (8
// channels) of token tau sits at c ^ (tau & (PPR - 1)); in vdec the 4-token
// quad s of channel ch sits at s ^ ((ch / DV) & 15). Both swizzles spread the
// 16 lanes of a compute read over all banks.
template <int KIND, int D>
__device__ __forceinline__ void pf_decode(const uint8_t* slot, uint8_t* kdec, uint8_t* vdec) {
  using G_ = Geo<KIND, D>;
  using F_ = PfGeo<KIND, D>;
  constexpr int NDW = F_::BPE / 4;
  constexpr int PLANE = kPfTokens * G_::RB;
  for (int blk = threadIdx.x; blk < (kPfTokens / 4) * F_::PPR; blk += 64 * kPfWaves) {
    const int tb = blk / F_::PPR, cb = blk % F_::PPR;
    const int byte = cb * F_::BPE;
    h2 vv[4][4];  // V of token i: channel pairs (2m, 2m + 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tau = 4 * tb + i;
      const int off = tau * G_::RB + 16 * ((byte / 16) ^ (tau & (G_::CPR - 1))) + byte % 16;
      uint32_t kw[NDW], vw[NDW];
#pragma unroll
      for (int d = 0; d < NDW; ++d) {
        kw[d] = *reinterpret_cast<const uint32_t*>(slot + off + 4 * d);
        vw[d] = *reinterpret_cast<const uint32_t*>(slot + PLANE + off + 4 * d);
      }
      _Float16 kh[8], vh[8];  // natural channel order
      {
        _Float16 tk[2 * Kv<KIND>::kPairsPerDword * NDW], tv[2 * Kv<KIND>::kPairsPerDword * NDW];
        decode_run<KIND, NDW>(kw, tk);
        decode_run<KIND, NDW>(vw, tv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kh[run_elem<KIND>(e)] = tk[e];
          vh[run_elem<KIND>(e)] = tv[e];
        }
      }
      h8 kop;
#pragma unroll
      for (int e = 0; e < 8; ++e) kop[e] = kh[e];
      *reinterpret_cast<h8*>(kdec + tau * (D * 2) + 16 * (cb ^ (tau & (F_::PPR - 1)))) = kop;
#pragma unroll
      for (int m = 0; m < 4; ++m) vv[i][m] = h2{vh[2 * m], vh[2 * m + 1]};
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = 8 * cb + c;
      const h4 quad = {vv[0][c / 2][c % 2], vv[1][c / 2][c % 2], vv[2][c / 2][c % 2],
                       vv[3][c / 2][c % 2]};
      *reinterpret_cast<h4*>(vdec + ch * (kPfTokens * 2) +
                             8 * (tb ^ ((ch / Geo<KIND, D>::DV) & 15))) = quad;
    }
  }
}

// Q of rows [row0, row0 + 32) of sequence b for KV head hk, in natural channel
// order (k-step ks, lane group g: channels 32 ks + 8 g .. + 7), folded with a
// PER_CHANNEL K scale as in start_run; resets the softmax state.
template <int KIND, int D, int QF>
__device__ __forceinline__ void pf_start_run(const AttnParams& p, int b, int row0, int hk, int L,
                                             float inv_m, float sgn,
                                             WaveState<KIND, D, 2, QF>& w) {
  using G_ = Geo<KIND, D>;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = row0 + 16 * rt + n;
    const bool rv = r < p.R;
    const int i = r / p.G, hg = r % p.G;
    const uint16_t* qrow = p.q + (((size_t)b * p.next_n + i) * p.Hq + hk * p.G + hg) * D;
#pragma unroll
    for (int ks = 0; ks < G_::KS; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      float xv[8];
      load_q8(qrow + d0, p.q_bf16, rv, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = xv[e];
        if constexpr (qf_fold(QF)) {
          const float xf = x * (p.k_scale[hk * D + d0 + e] * inv_m) * sgn;
          const _Float16 hi = (_Float16)xf;
          w.qa[rt][ks][e] = hi;
          w.qb[rt][ks][e] = (_Float16)(xf - (float)hi);
        } else {
          w.qa[rt][ks][e] = (_Float16)(x * sgn);
        }
      }
    }
    w.m_run[rt] = -INFINITY;
    w.l_acc[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < G_::DV; ++q) w.o[rt][q] = f4{0.f, 0.f, 0.f, 0.f};
    w.lim[rt] = p.causal ? (L - p.next_n + i) : 0x7fffffff;
  }
}

// Softmax step over a pair of 16-token tiles (sa: tokens 4g + e, sb: tokens
// 16 + 4g + e of the pair): P of the pair as two k = 32 operands, the fp16
// high parts (ph) and the fp16 remainders (pl), token order
// {4g .. 4g + 3, 16 + 4g .. 16 + 4g + 3} in lane group g. The weights carry the
// factor 2^kPScale, as in tile_softmax.
template <bool MASK>
__device__ __forceinline__ void pair_softmax(const f4 sa, const f4 sb, uint32_t okbits, float c2,
                                             float& m_run, float& alpha, bool& rescale, h8& ph,
                                             h8& pl) {
  float s[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (MASK) mx = (okbits >> e) & 1u ? fmaxf(mx, s[e]) : mx;
    else mx = fmaxf(mx, s[e]);
  }
  mx = rows_max(mx);
  const float m_old = m_run;
  const float m_new = fmaxf(m_old, mx);
  alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_old - m_new) * c2);
  rescale |= m_old != m_new && m_old != -INFINITY;
  const float mc = m_new == -INFINITY ? 0.f : m_new * c2 - kPScale;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float pf = __builtin_amdgcn_exp2f(fmaf(s[e], c2, -mc));
    if constexpr (MASK) pf = (okbits >> e) & 1u ? pf : 0.f;
    const _Float16 hi = (_Float16)pf;
    ph[e] = hi;
    pl[e] = p_lo(pf, hi);
  }
  m_run = m_new;
}

// A pair of 16-token sub-tiles (stage tokens 32 u .. 32 u + 31, sequence
// tokens t0 ..) for the wave's 32 rows from the decoded stage; P V and the row
// sums run as k = 32 products over the pair, once with P's high parts and once
// with its remainders. full: every row sees all 32 tokens.
template <int KIND, int D, int QF>
__device__ __forceinline__ void pf_pair(const uint8_t* kdec, const uint8_t* vdec, int u, int t0,
                                        int L, bool full, float c2,
                                        WaveState<KIND, D, 2, QF>& w) {
  using G_ = Geo<KIND, D>;
  using F_ = PfGeo<KIND, D>;
  constexpr int KS = G_::KS, DV = G_::DV;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  f4 sacc[2][2];  // [tile][row tile]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tau = 32 * u + 16 * h + n;
    h8 kop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kop[ks] = *reinterpret_cast<const h8*>(kdec + tau * (D * 2) +
                                             16 * ((4 * ks + g) ^ (tau & (F_::PPR - 1))));
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], w.qa[rt][ks], acc, 0, 0, 0);
        if constexpr (qf_fold(QF))
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], w.qb[rt][ks], acc, 0, 0, 0);
      }
      sacc[h][rt] = acc;
    }
  }
  h8 ph[2], pl[2];
  bool rescale = false;
  float alpha[2];
  if (full) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      pair_softmax<false>(sacc[0][rt], sacc[1][rt], 0xFFu, c2, w.m_run[rt], alpha[rt], rescale,
                          ph[rt], pl[rt]);
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      uint32_t okbits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
        okbits |= (uint32_t)(t < L && t <= w.lim[rt]) << e;
      }
      pair_softmax<true>(sacc[0][rt], sacc[1][rt], okbits, c2, w.m_run[rt], alpha[rt], rescale,
                         ph[rt], pl[rt]);
    }
  }
  if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int q = 0; q < DV; ++q) w.o[rt][q] *= alpha[rt];
      w.l_acc[rt] *= alpha[rt];
    }
  }
  // O^T += V^T P^T: channel row n * DV + q, the pair's tokens in P's order.
  // Decoded V of tokens past the end (tail slots may hold NaN codes) is
  // cleared by select before it can meet p = 0.
#pragma unroll
  for (int q = 0; q < DV; ++q) {
    const int ch = n * DV + q;
    const uint8_t* row = vdec + ch * (kPfTokens * 2);
    const h4 va0 = *reinterpret_cast<const h4*>(row + 8 * ((8 * u + g) ^ (ch / DV & 15)));
    const h4 va1 = *reinterpret_cast<const h4*>(row + 8 * ((8 * u + 4 + g) ^ (ch / DV & 15)));
    h8 va = {va0[0], va0[1], va0[2], va0[3], va1[0], va1[1], va1[2], va1[3]};
    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
        va[e] = t < L ? va[e] : (_Float16)0.0f;
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      w.o[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph[rt], w.o[rt][q], 0, 0, 0);
      w.o[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl[rt], w.o[rt][q], 0, 0, 0);
    }
  }
  const h8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                   (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    w.l_acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, ph[rt], w.l_acc[rt], 0, 0, 0);
    w.l_acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pl[rt], w.l_acc[rt], 0, 0, 0);
  }
}

template <int KIND, int D, int QF>
__global__ __launch_bounds__(64 * kPfWaves) void attn_prefill_kernel(
    AttnParams p, const int32_t* __restrict__ table, const int32_t* __restrict__ lens) {
  using G_ = Geo<KIND, D>;
  using F_ = PfGeo<KIND, D>;
  static_assert(F_::OK, "prefill layout does not fit this kind and head_dim");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[F_::LDS];
  uint8_t* ring = lds;
  uint8_t* kdec = lds + kPfStages * F_::STAGE;
  uint8_t* vdec = kdec + F_::KDEC;
  int* xi = reinterpret_cast<int*>(kdec);  // the scan result, read before any decode
  const int lane = threadIdx.x & 63, wv = uni(threadIdx.x >> 6);
  const float ks_tensor = (!qf_fold(QF) && p.k_scale_mode == PA_SCALE_PER_TENSOR) ? p.k_scale[0] : 1.0f;
  if (wv == 0) range_scan(p, lens, xi);
  __syncthreads();
  const int nitems = uni(xi[0]);
  if (nitems <= 0) return;
  ItemPos cp;
  cp.b = uni(xi[1]);
  cp.L = uni(xi[4]);
  cp.rb = uni(xi[5]);
  cp.nst = run_stages(p, cp.L, cp.rb);
  cp.hg = uni(xi[2]);
  cp.k = uni(xi[3]);
  __syncthreads();  // xi lives in kdec

  LoadPlan<KIND, D> lp;
  make_load_plan<KIND, D>(p, lp);

  // rows of this wave inside its run's group, and the steps they span
  auto row0_of = [&](int rb) { return rb * p.rpb + 32 * wv; };
  WaveState<KIND, D, 2, QF> w;

  // ---- prologue: items 0 and 1 in flight, the pages of item 2 looked up ----
  ItemPos pos[kPfStages];
  pos[0] = cp;
#pragma unroll
  for (int j = 1; j < kPfStages; ++j) {
    pos[j] = pos[j - 1];
    if (j - 1 < nitems) item_next(p, lens, pos[j]);
  }
  PageSet pgs[kPfStages - 1];
#pragma unroll
  for (int j = 0; j < kPfStages - 1; ++j) {
    const ItemPos& q = j < nitems ? pos[j] : pos[0];
    load_pages<KIND, D>(p, table, q, lp, pgs[j]);
  }
#pragma unroll
  for (int j = 0; j < kPfStages - 1; ++j)
    issue_stage<KIND, D>(p, pos[j], pgs[j], j < nitems, lp, ring + j * F_::STAGE);
  ItemPos ld = pos[kPfStages - 1];
  PageSet pg;
  if (kPfStages - 1 < nitems) load_pages<KIND, D>(p, table, ld, lp, pg);

  // scale constants and the first run's Q', behind the ring's first loads
  float qk, inv_m = 0.f;
  if constexpr (qf_fold(QF)) {
    float mx = 0.f;
    const int nks = p.Hkv * D;
    for (int i0 = 0; i0 < nks; i0 += 512) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + 64 * u + lane;
        v[u] = i < nks ? p.k_scale[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) mx = fmaxf(mx, fabsf(v[u]));
    }
    mx = wave_max(mx);
    inv_m = mx > 0.f ? 1.0f / mx : 0.f;
    qk = p.softmax_scale * mx;
  } else {
    qk = p.softmax_scale * ks_tensor;
  }
  const float sgn = qk < 0.f ? -1.f : 1.f;
  const float c2 = fabsf(qk) * kLog2e;
  pf_start_run<KIND, D, QF>(p, cp.b, row0_of(cp.rb), cp.hg, cp.L, inv_m, sgn, w);

  for (int j = 0; j < nitems; ++j) {
    // item j has landed for every wave, and every wave is done with the
    // decoded copy of item j - 1
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kPfStages - 2) * G_::NL) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int jn = j + kPfStages - 1;
    const bool live_n = jn < nitems;
    issue_stage<KIND, D>(p, ld, pg, live_n, lp, ring + (jn % kPfStages) * F_::STAGE);
    if (live_n) item_next(p, lens, ld);
    pf_decode<KIND, D>(ring + (j % kPfStages) * F_::STAGE, kdec, vdec);
    lds_barrier();
    // this wave's rows: steps i_first .. i_last
    const int r0 = row0_of(cp.rb);
    if (r0 < p.R) {
      const int i_first = r0 / p.G, i_last = (min(r0 + 32, p.R) - 1) / p.G;
      const int vis = p.causal ? max(0, min(cp.L, cp.L - p.next_n + i_last + 1)) : cp.L;
      const int flim = cp.L - (p.causal ? p.next_n - 1 - i_first : 0);
      const int tbase = cp.k * kPfTokens;
      for (int u = 0; u < kPfTokens / 32; ++u) {
        const int t0 = tbase + 32 * u;
        if (t0 >= vis) break;
        pf_pair<KIND, D, QF>(kdec, vdec, u, t0, cp.L, t0 + 32 <= flim, c2, w);
      }
    }
    // end of a run inside this range: write the wave's rows of its partial
    const int b = cp.b, hg = cp.hg, rb = cp.rb;
    item_next(p, lens, cp);
    if (j + 1 == nitems || cp.b != b || cp.hg != hg || cp.rb != rb) {
      const int run = (b * p.nrb + rb) * p.hgroups + hg;
      if (row0_of(rb) < p.R)
        write_partial<KIND, D, 2, QF>(p, part_index(p, run, blockIdx.x, 0), c2, w,
                                        32 * wv);
      if (j + 1 < nitems)
        pf_start_run<KIND, D, QF>(p, cp.b, row0_of(cp.rb), cp.hg, cp.L, inv_m, sgn, w);
    }
    if (jn + 1 < nitems) load_pages<KIND, D>(p, table, ld, lp, pg);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

typedef void (*PrefillFn)(AttnParams, const int32_t*, const int32_t*);

template <int KIND, int D>
PrefillFn pick_prefill_d(bool fold) {
  if constexpr (!PfGeo<KIND, D>::OK) {
    return nullptr;
  } else {
    if (fold) {
      if constexpr (KIND == PA_KV_F16 || KIND == PA_KV_BF16) return nullptr;
      else return attn_prefill_kernel<KIND, D, kQSplit>;
    }
    return attn_prefill_kernel<KIND, D, kQPlain>;
  }
}

template <int KIND>
PrefillFn pick_prefill(int D, bool fold) {
  if constexpr (KIND != PA_KV_INT4)
    if (D == 64) return pick_prefill_d<KIND, 64>(fold);
  if (D == 128) return pick_prefill_d<KIND, 128>(fold);
  return nullptr;
}

typedef void (*RingFn)(AttnParams, const int32_t*, const int32_t*, const uint32_t*);

// The ring kernel of one Q' format (kQPlain / kQSplit / kQPacked / kQDup) and
// row-tile count. The folded formats exist for scaled kinds only, the packed
// ones for one row tile, and the row-block mode has two row tiles.
template <int KIND, int D, int NWB, int MODE>
RingFn pick_qf(int RT, int qf) {
  constexpr bool kFold = KIND != PA_KV_F16 && KIND != PA_KV_BF16;
  if constexpr (MODE != kModeRows) {
    if (RT == 1) {
      if (qf == kQPlain) return attn_ring_kernel<KIND, D, 1, kQPlain, NWB, MODE>;
      if (qf == kQDup) return attn_ring_kernel<KIND, D, 1, kQDup, NWB, MODE>;
      if constexpr (kFold) {
        if (qf == kQSplit) return attn_ring_kernel<KIND, D, 1, kQSplit, NWB, MODE>;
        if (qf == kQPacked) return attn_ring_kernel<KIND, D, 1, kQPacked, NWB, MODE>;
      }
      return nullptr;
    }
  }
  if (RT == 2) {
    if (qf == kQPlain) return attn_ring_kernel<KIND, D, 2, kQPlain, NWB, MODE>;
    if constexpr (kFold)
      if (qf == kQSplit) return attn_ring_kernel<KIND, D, 2, kQSplit, NWB, MODE>;
  }
  return nullptr;
}

// NWB: the launch bound in waves (4 or 8); a 4-wave workgroup gets twice the
// registers per wave. Row tiles RT are 1 or 2 (16 or 32 rows): more rows come
// in row blocks of 32 (kModeRows).
template <int KIND, int D, int NWB>
RingFn pick_rt(int RT, int qf, int mode) {
  if (mode == kModeSparse) return pick_qf<KIND, D, NWB, kModeSparse>(RT, qf);
  if (mode == kModeRows) return pick_qf<KIND, D, NWB, kModeRows>(RT, qf);
  return pick_qf<KIND, D, NWB, kModeDense>(RT, qf);
}

template <int KIND, int D>
RingFn pick_nw(int nw, int RT, int qf, int mode) {
  return nw <= 4 ? pick_rt<KIND, D, 4>(RT, qf, mode) : pick_rt<KIND, D, 8>(RT, qf, mode);
}

template <int KIND>
RingFn pick_d(int D, int nw, int RT, int qf, int mode) {
  if constexpr (KIND != PA_KV_INT4)
    if (D == 64) return pick_nw<KIND, 64>(nw, RT, qf, mode);
  if (D == 128) return pick_nw<KIND, 128>(nw, RT, qf, mode);
  return pick_nw<KIND, 256>(nw, RT, qf, mode);
}

// Ring kernel of one KV kind (each defined in its own translation unit).
RingFn pick_ring_f16(int D, int nw, int RT, int qf, int mode);
RingFn pick_ring_bf16(int D, int nw, int RT, int qf, int mode);
RingFn pick_ring_e4m3(int D, int nw, int RT, int qf, int mode);
RingFn pick_ring_int8(int D, int nw, int RT, int qf, int mode);
RingFn pick_ring_int4(int D, int nw, int RT, int qf, int mode);
PrefillFn pick_prefill_f16(int D, bool fold);
PrefillFn pick_prefill_bf16(int D, bool fold);
PrefillFn pick_prefill_e4m3(int D, bool fold);
PrefillFn pick_prefill_int8(int D, bool fold);
PrefillFn pick_prefill_int4(int D, bool fold);

}  // namespace pa
