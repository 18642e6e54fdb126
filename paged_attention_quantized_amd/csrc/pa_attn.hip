// pa_attn.hip -- paged attention over a quantized KV cache on gfx950.
//
// Work decomposition. The KV reduction is cut into "items": TS consecutive
// logical tokens of one sequence for one group of HPU KV heads. Items are
// ordered by (sequence, head group, logical position) and the persistent grid
// (one workgroup per compute unit) gives each workgroup a contiguous item
// range of equal cost: every item costs one slot and every (sequence, head
// group) run start run_cost more (the q reload and partial store there drain
// the load pipeline), and workgroup w takes the items in slots
// [w*Q, (w+1)*Q), Q = ceil(slots / workgroups). Every workgroup therefore gets
// about the same streaming time whatever the mix of context lengths, and all
// cut points depend on logical positions only, never on physical block ids
// [RELOC, Summary].
//
// Memory path. A workgroup streams its items through a ring of kStages stages
// in LDS. A stage holds the item's TS tokens x HPU heads of K and V, fetched
// with global_load_lds_dwordx4 (HBM -> LDS, no registers), and is cut into one
// region per wave: each wave loads the K rows, then the V rows, of exactly the
// 16 tokens and the head it computes, so it waits for its own loads only (an
// explicit vmcnt) and the ring needs no barrier between waves. kStages - 1
// stages are in flight while one is computed, and every step issues the same
// number of loads (past the end: dummy in-bounds loads into the free slot) so
// the count stays exact. A wave's 16 tokens lie in one page: one block-table
// lookup per item, a scalar load issued one step ahead, so no vector load
// waits behind the ring. Within a row, 16-byte pieces are stored XOR-swizzled
// by the row index to spread LDS banks. (The prefill kernel below shares one
// decoded copy of each stage between its waves and keeps a workgroup-wide
// layout with barriers.) Tokens past the
// sequence end are read only inside real pages; pages past the end are never
// read (their lanes re-read the stage's first page), which keeps the null
// block 0 unread [NULLPAD, Root cause].
//
// Compute. Wave w of the workgroup serves head hl = w % HPU of the group and
// the 16-token sub-tile st = w / HPU of every stage:
//   1. K codes from LDS -> fp16 (exact for E4M3/INT8/INT4), S^T = K Q'^T with
//      v_mfma_f32_16x16x32_f16 (tokens x query rows); a PER_CHANNEL K scale is
//      folded into Q' = q * k_scale / max|k_scale| as fp16 hi + lo parts
//      (both in one operand's 16 columns when a KV head has at most 8 query
//      rows) and max|k_scale| goes into the score scale [FOLD, Approach],
//   2. online softmax in base 2 on raw scores; tokens past the end or past a
//      row's causal limit are selected to p = 0 (never multiplied),
//   3. V codes from LDS -> fp16, rows of invalid tokens zeroed by select
//      [NULLPAD, Fix], O^T += V^T P^T with v_mfma_f32_16x16x16_f16.
// At the end of each (sequence, head group) run inside its range the waves of
// a head fold their sub-tile states in LDS (sub-tile order) and the first
// writes (m, l, c) and unnormalized O as the workgroup's partial; the merge
// kernel combines the partials of a (sequence, KV head) in workgroup order
// and applies v_scale / l.
//
// Query rows. Up to 32 rows per KV head (next_n x q heads per KV head) sit in
// one or two 16-row MFMA tiles of every wave. More rows are cut into row
// blocks, each a run of its own on the cost line that walks only the tokens
// its last row can see: blocks of 32 rows in the ring kernel, or, from 128
// rows where it fits, 256-row groups in the prefill kernel, whose 8 waves are
// the 8 row blocks of one KV head sharing each stage decoded once into fp16.
//
// Selection-driven sparse attention. A planner kernel turns each sequence's
// selected token ids into a union of logical pages in ascending order with
// one token mask per query row; the ring kernel then walks that plan as its
// block table, one page per item, and keeps for each row exactly the tokens
// its mask selects [RELOC] [NULLPAD].
#include <math.h>

#include <atomic>

#include "pa_attn.hpp"
#include "pa_host.hpp"

namespace pa {

// Combine the partials of each (sequence b, KV head hk, query row) in a fixed
// order (workgroup order), which depends on logical positions only
// [RELOC], and apply the V scale and 1/l. A row with no visible token is +0.
// One thread per 4 output channels; the item ranges of the ring kernel follow
// from the sequence starts it published.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p, int D) {
  const int bh = blockIdx.x;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int hg = hk >> p.lhpu, hl = hk & (p.hpu - 1);
  const int idx = blockIdx.y * 256 + threadIdx.x;
  // the ring kernel's split: item k of run (b, rb, hg) sits at cost slot
  // first_slot(b) + (slots of row blocks before rb) + hg * (nst + run_cost) +
  // run_cost + k, and workgroup w owns slots [w * qc, (w + 1) * qc)
  const int qc = max(1, (p.ws_seq[p.B] + p.nwg - 1) / p.nwg);
  const int L = p.context_lens[b];
  const int r = 4 * idx / D, d = 4 * idx % D;
  // a workgroup's 1024 / D rows never straddle a row block (32 rows, or all
  // R rows when there is one block): its block is workgroup-uniform, and the
  // slots of the blocks before it are summed 64 blocks at a time
  const int rb = uni((int)blockIdx.y * (1024 / D) / p.rpb), rl = r - rb * p.rpb;
  int before = 0;
  for (int x0 = 0; x0 < rb; x0 += 64) {
    const int x = x0 + (int)(threadIdx.x & 63);
    const int n = x < rb ? run_stages(p, L, x) : 0;
    before += lane_val(wave_incl_scan(n > 0 ? p.hgroups * (n + p.run_cost) : 0), 63);
  }
  int slot0 = p.ws_seq[b] + uni(before);
  if (4 * idx >= p.R * D) return;  // after the wave-wide sums, which need every lane
  const int nst = run_stages(p, L, rb);
  slot0 += hg * (nst + p.run_cost) + p.run_cost;
  const int i = r / p.G, h = hk * p.G + r % p.G;
  float m = -INFINITY, l = 0.f;
  f4 o = {0.f, 0.f, 0.f, 0.f};
  if (nst > 0) {
    const int w_first = slot0 / qc, w_last = (slot0 + nst - 1) / qc;
    const int run = (b * p.nrb + rb) * p.hgroups + hg;
    const int nparts = w_last - w_first + 1;
    constexpr int U = 8;
    for (int k0 = 0; k0 < nparts; k0 += U) {
      f4 rec[U], x[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (k0 + k < nparts) {
          const int part = k0 + k;
          const size_t u = part_index(p, run, w_first + part, hl);
          rec[k] = p.ws_ml[u * p.rpb + rl];
          x[k] = *reinterpret_cast<const f4*>(p.ws_o + (u * p.rpb + rl) * D + d);
        } else {
          rec[k] = f4{-INFINITY, 0.f, 0.f, 0.f};
          x[k] = f4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (rec[k][0] == -INFINITY) continue;  // a partial that saw no token
        const float cc = rec[k][2];
        const float mn = fmaxf(m, rec[k][0]);
        const float a = m == -INFINITY ? 0.f : exp2f((m - mn) * cc);
        const float bw = exp2f((rec[k][0] - mn) * cc);
        l = l * a + rec[k][1] * bw;
        o = o * a + x[k] * bw;
        m = mn;
      }
    }
  }
  f4 val = l > 0.f ? o / l : f4{0.f, 0.f, 0.f, 0.f};
  if (p.v_scale_mode == PA_SCALE_PER_TENSOR) {
    val *= p.v_scale[0];
  } else if (p.v_scale_mode == PA_SCALE_PER_CHANNEL) {
    const float* vs = p.v_scale + hk * D + d;
    val *= f4{vs[0], vs[1], vs[2], vs[3]};
  }
  const size_t at = (((size_t)b * p.next_n + i) * p.Hq + h) * D + d;
  if (p.out_bf16) {
    // round to nearest even on the fp32 bits (no NaN can reach here: a NaN
    // keeps a quiet payload)
    uint16_t hb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = __float_as_uint(val[e]);
      hb[e] = val[e] != val[e] ? (uint16_t)((u >> 16) | 0x40u)
                               : (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    *reinterpret_cast<u2*>(static_cast<uint16_t*>(p.out) + at) =
        u2{hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16)};
  } else {
    *reinterpret_cast<h4*>(static_cast<_Float16*>(p.out) + at) =
        h4{(_Float16)val[0], (_Float16)val[1], (_Float16)val[2], (_Float16)val[3]};
  }
}

// Plan probe: what the attention kernels walk. Workgroup w of the persistent
// grid runs the kernels' own range scan and writes each item of its range,
// in walking order, at its global index: {w, sequence, row block, head group,
// first logical token, physical block of the item's first page}. Workgroup 0
// also leaves every sequence's first cost slot (the merge's arithmetic) in
// p.ws_seq and the item total in *total.
__global__ __launch_bounds__(64) void plan_probe_kernel(AttnParams p, int32_t* items,
                                                        int64_t cap, int32_t* total) {
  __shared__ int xi[8];
  range_scan(p, p.context_lens, xi);
  if (blockIdx.x == 0) {
    // the item total, by the cost-line bookkeeping the kernels use
    int n_all = 0;
    for (int base = 0; base < p.B; base += 64) {
      const int b = base + (int)threadIdx.x;
      int cost, items;
      seq_cost(p, b < p.B ? p.context_lens[b] : 0, cost, items);
      n_all += lane_val(wave_incl_scan(items), 63);
    }
    if (threadIdx.x == 0) *total = n_all;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int n = xi[0], ia = xi[6];
  ItemPos it;
  it.b = xi[1];
  it.hg = xi[2];
  it.k = xi[3];
  it.L = xi[4];
  it.rb = xi[5];
  it.nst = run_stages(p, it.L, it.rb);
  for (int j = 0; j < n && ia + j < cap; ++j) {
    const int t0 = it.k << p.lts;
    int32_t* e = items + (size_t)(ia + j) * 6;
    e[0] = blockIdx.x;
    e[1] = it.b;
    e[2] = it.rb;
    e[3] = it.hg;
    e[4] = t0;
    e[5] = p.block_table[(size_t)it.b * p.max_blocks + (t0 >> p.lbs)];
    item_next(p, p.context_lens, it);
  }
}

// Grouped union planner of a selection [RELOC, Summary: a physical-page union
// with token masks, ordered with the logical page as the key and the physical
// block as payload]. One 1024-thread workgroup per sequence b: every valid
// selected token (0 <= t < L_b) sets the bit of its logical page in an LDS
// bitmap; a wave scan of the word popcounts ranks the pages in logical order;
// entry e gets {block_table[b, page], page}; the row masks are ORed together
// in LDS (bit t % bs of word (e(t), row)) and written out coalesced, in chunks
// of entries when cap * next_n exceeds the LDS buffer. Every selection pass
// issues all of a thread's loads before it uses any. Writes count[b]
// (entries) and vlen[b] = count * bs when those pointers are set; entries for
// e < count, masks for all e < cap.
constexpr int kPlanThreads = 1024;
constexpr int kPlanUnroll = 8;         // selection entries per thread per pass
constexpr int kPlanMaskWords = 8192;   // LDS mask words per chunk of entries

__device__ __forceinline__ void plan_load_sel(const int32_t* __restrict__ srow, int nsel, int base,
                                              int32_t (&tv)[kPlanUnroll]) {
#pragma unroll
  for (int u = 0; u < kPlanUnroll; ++u) {
    const int x = base + u * kPlanThreads + (int)threadIdx.x;
    tv[u] = x < nsel ? srow[x] : -1;
  }
}

__global__ __launch_bounds__(kPlanThreads) void sparse_plan_kernel(
    const int32_t* __restrict__ sel, int topk, const int32_t* __restrict__ table,
    const int32_t* __restrict__ lens, int max_blocks, int lbs, int next_n, int cap,
    int32_t* __restrict__ entries, uint32_t* __restrict__ masks, int32_t* count, int32_t* vlen) {
  __shared__ uint32_t bm[kPlanWords];
  __shared__ int wrank[kPlanWords];
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ uint32_t mbuf[kPlanMaskWords];
  static_assert(kPlanWords <= kPlanThreads, "one bitmap word per thread in the rank scan");
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bs = 1 << lbs;
  // tokens past the table's pages are never selectable (keeps the bitmap in bounds)
  const int L = min(lens[b], max_blocks << lbs);
  const int npages = L > 0 ? (L + bs - 1) >> lbs : 0;
  const int nw = (npages + 31) >> 5;
  const int nsel = next_n * topk;
  const int32_t* srow = sel + (size_t)b * nsel;
  if (tid < kPlanWords) bm[tid] = 0u;
  __syncthreads();
  for (int base = 0; base < nsel; base += kPlanUnroll * kPlanThreads) {
    int32_t tv[kPlanUnroll];
    plan_load_sel(srow, nsel, base, tv);
#pragma unroll
    for (int u = 0; u < kPlanUnroll; ++u)
      if (tv[u] >= 0 && tv[u] < L) {
        const int lp = tv[u] >> lbs;
        atomicOr(&bm[lp >> 5], 1u << (lp & 31));
      }
  }
  __syncthreads();
  // exclusive rank of bitmap word tid: wave scans, then the wave totals
  const int c = tid < nw ? __popc(bm[tid]) : 0;
  const int incl = wave_incl_scan(c);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kPlanThreads / 64; ++i) {
    off += i < wv ? wsum[i] : 0;
    total += wsum[i];
  }
  if (tid < kPlanWords) wrank[tid] = off + incl - c;
  __syncthreads();
  // entries: one thread per logical page
  for (int lp = tid; lp < npages; lp += kPlanThreads) {
    const uint32_t word = bm[lp >> 5];
    if ((word >> (lp & 31)) & 1u) {
      const int e = wrank[lp >> 5] + __popc(word & ((1u << (lp & 31)) - 1u));
      if (e < cap) {
        const size_t at = (size_t)b * cap + e;
        entries[2 * at + 0] = table[(size_t)b * max_blocks + lp];
        entries[2 * at + 1] = lp;
      }
    }
  }
  // row masks, a chunk of entries at a time
  const int n = total < cap ? total : cap;
  const int cw = kPlanMaskWords / next_n;
  for (int e0 = 0; e0 < cap; e0 += cw) {
    const int ne = min(cw, cap - e0);
    for (int x = tid; x < ne * next_n; x += kPlanThreads) mbuf[x] = 0u;
    __syncthreads();
    if (e0 < n) {
      for (int base = 0; base < nsel; base += kPlanUnroll * kPlanThreads) {
        int32_t tv[kPlanUnroll];
        plan_load_sel(srow, nsel, base, tv);
#pragma unroll
        for (int u = 0; u < kPlanUnroll; ++u) {
          const int t = tv[u];
          if (t >= 0 && t < L) {
            const int lp = t >> lbs, w = lp >> 5;
            const int e = wrank[w] + __popc(bm[w] & ((1u << (lp & 31)) - 1u)) - e0;
            const int row = (base + u * kPlanThreads + tid) / topk;
            if (e >= 0 && e < ne) atomicOr(&mbuf[e * next_n + row], 1u << (t & (bs - 1)));
          }
        }
      }
    }
    __syncthreads();
    uint32_t* mrow = masks + ((size_t)b * cap + e0) * next_n;
    for (int x = tid; x < ne * next_n; x += kPlanThreads) mrow[x] = mbuf[x];
    __syncthreads();
  }
  if (tid == 0) {
    if (count) count[b] = n;
    if (vlen) vlen[b] = n * bs;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

struct Shape {
  int R, RT, RB, hpu, hgroups, ts, nw, nsub, nwg;
  int nrb, rpb;                          // query row blocks and rows per block
  int sparse, sp_cap;                    // selection-driven mode: plan entries per sequence
  int prefill;                           // the prefill layout (attn_prefill_kernel)
  size_t sp_entries_bytes, sp_masks_bytes, sp_vlen_bytes;
  int wgmerge;
  int run_cost;                          // cost-line slots of a run start
  int64_t parts;
  size_t ml_bytes, o_bytes, seq_bytes;
};

int gcd_int(int x, int y) { return y == 0 ? x : gcd_int(y, x % y); }

int ilog2(int x) {  // x is a power of two
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

PrefillFn pick_prefill_fn(int kind, int D, bool fold) {
  switch (kind) {
    case PA_KV_F16: return pick_prefill_f16(D, fold);
    case PA_KV_BF16: return pick_prefill_bf16(D, fold);
    case PA_KV_E4M3: return pick_prefill_e4m3(D, fold);
    case PA_KV_INT8: return pick_prefill_int8(D, fold);
    case PA_KV_INT4: return pick_prefill_int4(D, fold);
  }
  return nullptr;
}

pa_status check_args(const pa_attn_args* a, Shape* sh, bool need_ptrs, int sparse_topk = -1) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "paged_attn: args is NULL");
  if (a->batch < 0 || a->next_n < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1 ||
      a->max_context_len < 0 || a->max_blocks_per_seq < 1 || a->num_blocks < 1)
    return fail(PA_ERR_INVALID_ARG, "paged_attn: negative or zero size");
  if (a->num_q_heads % a->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "paged_attn: num_q_heads %% num_kv_heads != 0");
  if (!valid_kind(a->kv_kind) || !valid_mode(a->k_scale_mode) || !valid_mode(a->v_scale_mode))
    return fail(PA_ERR_INVALID_ARG, "paged_attn: unknown kv_kind or scale mode");
  if (a->q_dtype != PA_DT_F16 && a->q_dtype != PA_DT_BF16)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: q_dtype must be F16 or BF16");
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: head_dim must be 64, 128 or 256");
  if (a->block_size != 16 && a->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: block_size must be 16 or 32");
  const int rb = a->head_dim * kv_bits(a->kv_kind) / 8;
  if (rb % 64) return fail(PA_ERR_UNSUPPORTED, "paged_attn: head_dim too small for this kv kind");
  if ((a->kv_kind == PA_KV_F16 || a->kv_kind == PA_KV_BF16) &&
      (a->k_scale_mode != PA_SCALE_NONE || a->v_scale_mode != PA_SCALE_NONE))
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: F16 / BF16 KV takes no scales");
  if (a->softmax_scale < 0.f || !(a->softmax_scale == a->softmax_scale))
    return fail(PA_ERR_INVALID_ARG, "paged_attn: softmax_scale must be >= 0");
  const int G = a->num_q_heads / a->num_kv_heads;
  if (a->next_n > kMaxNextN || (int64_t)a->next_n * G > kMaxRows)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: next_n > %d or next_n * q heads per kv head > %d",
                kMaxNextN, kMaxRows);
  const int R = a->next_n * G;
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
  // at least kPfMinRows rows per KV head, where the layout fits: the prefill
  // kernel, 256-row groups of one head
  sh->prefill = sparse_topk < 0 && R >= kPfMinRows &&
                pick_prefill_fn(a->kv_kind, a->head_dim,
                                a->k_scale_mode == PA_SCALE_PER_CHANNEL) != nullptr;
  // more than 32 rows otherwise: blocks of 32 rows (two row tiles), one run each
  sh->rpb = sh->prefill ? 32 * kPfWaves : (R <= 32 ? R : 32);
  sh->nrb = (int)ceil_div(R, sh->rpb);
  sh->RT = sh->rpb <= 16 ? 1 : 2;  // the prefill kernel holds two row tiles per wave
  sh->RB = rb;
  // An item spans hpu KV heads (a divisor of the KV head count, at most 1 KiB
  // of row bytes per token) and ts tokens, so that one stage (K and V) is at
  // most 32 KiB and a workgroup has at most 8 waves of 16-token sub-tiles.
  int hpu = gcd_int(a->num_kv_heads, kMaxWaves);
  int ts;
  if (sparse_topk >= 0) {
    // selection-driven mode: an item is one page of the union plan
    if (a->next_n > kSparseRows || R > 32)
      return fail(PA_ERR_UNSUPPORTED, "paged_attn_sparse: next_n <= 4 and next_n * G <= 32");
    if ((int64_t)a->max_blocks_per_seq > 32 * kPlanWords)
      return fail(PA_ERR_UNSUPPORTED, "paged_attn_sparse: max_blocks_per_seq > 16384");
    ts = a->block_size;
    while (hpu > 1 && (2 * ts * hpu * rb > kStageMax || hpu * (ts / 16) > kMaxWaves)) hpu /= 2;
    if (2 * ts * hpu * rb > kStageMax)
      return fail(PA_ERR_UNSUPPORTED, "paged_attn_sparse: one page exceeds a ring stage");
  } else if (sh->prefill) {
    hpu = 1;
    ts = kPfTokens;
  } else {
    while (hpu > 1 && hpu * rb > 1024) hpu /= 2;
    // Two row tiles: a head's partial is 32 rows x D fp32, and every run
    // splits into about one partial per workgroup it crosses. At most 4 heads
    // per item doubles the runs (head groups) and halves the workgroups each
    // crosses, so the partials the ring writes and the merge reads halve; the
    // ring itself takes the same time (measured on the FP8 verify workload:
    // merge 13.6 -> ~7 us).
    if (sh->RT == 2 && hpu > 4) hpu = 4;
    ts = kStageMax / 2 / (hpu * rb);
    if (ts > 64) ts = 64;
    if (ts > 16 * kMaxWaves / hpu) ts = 16 * kMaxWaves / hpu;
    if (ts < 16) ts = 16;
  }
  sh->hpu = hpu;
  sh->hgroups = a->num_kv_heads / hpu;
  sh->ts = ts;
  sh->nsub = ts / 16;
  sh->nw = hpu * sh->nsub;
  // a wave's ring loads of an item touch at most two pages (the kernel looks
  // up two): with two or more waves they span 32 / hpu <= 2 * bs tokens, and a
  // single wave holds a whole item, so the item must fit two pages
  if (sh->nw == 1 && ts > 2 * a->block_size)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: item spans more than two pages");
  sh->nwg = device_cus();
  // Sub-tile states are merged inside the workgroup, one row tile of one head
  // at a time (in the MFMA layout: 16 rows x D fp32, plus m and l, through
  // the LDS exchange buffer), so every run leaves one partial per head and
  // workgroup.
  if (a->head_dim / 16 * 1024 + 512 > kXchBytes)
    return fail(PA_ERR_UNSUPPORTED, "paged_attn: head_dim too large for the LDS exchange");
  sh->wgmerge = sh->nsub > 1 ? 1 : 0;
  if (sh->prefill) sh->wgmerge = 1;  // one partial per group: the waves own disjoint rows
  // Cost of a run start in items, for the cost line: the first Q' loads wait
  // for every ring load in flight, the ring refills, the partial is written,
  // and with sub-tiles merged in the workgroup the LDS exchange runs. Measured
  // from per-workgroup finish times against the runs each range touches, then
  // tuned by timing: 2 items with one row tile and no exchange, 12 with two
  // row tiles, and with the exchange 4 items plus about half an item per
  // merged (head, extra sub-tile). The sparse route and the prefill layout
  // keep 2 (no measurable change between 2 and 8 for the sparse route).
  sh->run_cost = 2;
  if (sparse_topk < 0 && !sh->prefill)
    sh->run_cost = 2 + (sh->RT == 2 ? 10 : 0) +
                   (sh->wgmerge ? 4 + (sh->hpu * (sh->nsub - 1) + 1) / 2 : 0);
  // partial slots: one per (run, workgroup) pair a run can span, at most
  // runs + workgroups of them, each with one partial per head
  const int64_t slots = (int64_t)a->batch * sh->nrb * sh->hgroups + sh->nwg;
  sh->parts = slots * sh->hpu;
  sh->ml_bytes = (size_t)round_up(sh->parts * sh->rpb * 16, 256);
  sh->o_bytes = (size_t)round_up(sh->parts * sh->rpb * a->head_dim * 4, 256);
  // sequence first slots, then the PA_VALIDATE flags
  sh->seq_bytes = (size_t)round_up(((int64_t)a->batch + 1) * 4, 256) + kValidateBytes;
  sh->sparse = sparse_topk >= 0 ? 1 : 0;
  sh->sp_cap = 0;
  sh->sp_entries_bytes = sh->sp_masks_bytes = sh->sp_vlen_bytes = 0;
  if (sh->sparse) {
    const int64_t cap64 = (int64_t)a->next_n * sparse_topk;
    sh->sp_cap = (int)(cap64 < a->max_blocks_per_seq ? cap64 : a->max_blocks_per_seq);
    if (sh->sp_cap < 1) sh->sp_cap = 1;
    sh->sp_entries_bytes = (size_t)round_up((int64_t)a->batch * sh->sp_cap * 8, 256);
    sh->sp_masks_bytes = (size_t)round_up((int64_t)a->batch * sh->sp_cap * a->next_n * 4, 256);
    sh->sp_vlen_bytes = (size_t)round_up((int64_t)a->batch * 4, 256);
  }
  return PA_OK;
}

AttnParams make_params(const pa_attn_args* a, const Shape& sh, void* ws) {
  AttnParams p;
  p.out = a->out;
  p.q = (const uint16_t*)a->q;
  p.q_bf16 = a->q_dtype == PA_DT_BF16;
  p.out_bf16 = a->q_dtype == PA_DT_BF16;
  p.k_cache = (const uint8_t*)a->k_cache;
  p.v_cache = (const uint8_t*)a->v_cache;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.context_lens = a->context_lens;
  p.ws_ml = (f4*)ws;
  p.ws_o = (float*)((char*)ws + sh.ml_bytes);
  p.ws_seq = (int*)((char*)ws + sh.ml_bytes + sh.o_bytes);
  p.B = a->batch;
  p.next_n = a->next_n;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.R = sh.R;
  p.nrb = sh.nrb;
  p.rpb = sh.rpb;
  p.bs = a->block_size;
  p.max_blocks = a->max_blocks_per_seq;
  p.hpu = sh.hpu;
  p.hgroups = sh.hgroups;
  p.ts = sh.ts;
  p.nw = sh.nw;
  p.nsub = sh.nsub;
  p.nwg = sh.nwg;
  p.lbs = ilog2(a->block_size);
  p.lts = ilog2(sh.ts);
  p.lhpu = ilog2(sh.hpu);
  p.wgmerge = sh.wgmerge;
  p.run_cost = sh.run_cost;
  p.k_scale_mode = a->k_scale_mode;
  p.v_scale_mode = a->v_scale_mode;
  p.causal = a->causal ? 1 : 0;
  p.softmax_scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / sqrtf((float)a->head_dim);
  return p;
}

RingFn pick_ring(int kind, int D, int nw, int RT, int qf, int mode) {
  switch (kind) {
    case PA_KV_F16: return pick_ring_f16(D, nw, RT, qf, mode);
    case PA_KV_BF16: return pick_ring_bf16(D, nw, RT, qf, mode);
    case PA_KV_E4M3: return pick_ring_e4m3(D, nw, RT, qf, mode);
    case PA_KV_INT8: return pick_ring_int8(D, nw, RT, qf, mode);
    case PA_KV_INT4: return pick_ring_int4(D, nw, RT, qf, mode);
  }
  return nullptr;
}

// PA_VALIDATE=1 check of the call's context lengths and visible block ids; the
// flags live in the last kValidateBytes of the sequence-start region.
pa_status validate_attn(const char* who, const pa_attn_args* a, const Shape& sh, void* ws,
                        hipStream_t s) {
  int* flags = (int*)((char*)ws + sh.ml_bytes + sh.o_bytes + sh.seq_bytes - kValidateBytes);
  return validate_tables(who, a->block_table, a->context_lens, a->batch, a->max_blocks_per_seq,
                         a->max_context_len, a->block_size, a->num_blocks, true, flags, s);
}

// Q' format of the ring kernel: with at most 8 query rows per KV head the rows
// are mirrored in the operand's upper 8 columns (and P packed the same way);
// PER_CHANNEL K scales fold into hi + lo parts of Q'.
int q_format(const pa_attn_args* a, const Shape& sh) {
  const bool fold = a->k_scale_mode == PA_SCALE_PER_CHANNEL;
  const bool pack = sh.nrb == 1 && sh.RT == 1 && sh.rpb <= 8;
  return fold ? (pack ? kQPacked : kQSplit) : (pack ? kQDup : kQPlain);
}

// Enqueue the ring kernel and the merge for checked arguments.
pa_status launch_attn(const pa_attn_args* a, const Shape& sh, void* workspace, hipStream_t s) {
  const bool hilo = a->k_scale_mode == PA_SCALE_PER_CHANNEL;
  AttnParams p = make_params(a, sh, workspace);
  if (sh.prefill) {
    PrefillFn fn = pick_prefill_fn(a->kv_kind, a->head_dim, hilo);
    if (!fn) return fail(PA_ERR_UNSUPPORTED, "paged_attn: no prefill kernel for this kind/shape");
    launch_timed(fn, dim3((unsigned)sh.nwg), dim3(64 * kPfWaves), s, p, a->block_table,
                 a->context_lens);
  } else {
    RingFn fn = pick_ring(a->kv_kind, a->head_dim, sh.nw, sh.RT, q_format(a, sh),
                          sh.nrb > 1 ? kModeRows : kModeDense);
    if (!fn) return fail(PA_ERR_UNSUPPORTED, "paged_attn: no kernel for this kind/shape");
    launch_timed(fn, dim3((unsigned)sh.nwg), dim3(64 * sh.nw), s, p, a->block_table,
                 a->context_lens, (const uint32_t*)nullptr);
  }
  pa_status st = launch_status("paged_attn attention kernel");
  if (st != PA_OK) return st;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(a->batch * a->num_kv_heads),
                     (unsigned)ceil_div((int64_t)sh.R * a->head_dim / 4, 256)), dim3(256), 0, s,
                     p, a->head_dim);
  return launch_status("paged_attn merge kernel");
}

}  // namespace

}  // namespace pa

using namespace pa;

extern "C" size_t paged_attn_workspace_size(const pa_attn_args* a) {
  Shape sh;
  if (check_args(a, &sh, false) != PA_OK) return 0;
  return sh.ml_bytes + sh.o_bytes + sh.seq_bytes;
}

extern "C" pa_status paged_attn_fwd(const pa_attn_args* a, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Shape sh;
  pa_status st = check_args(a, &sh, true);
  if (st != PA_OK) return st;
  const size_t ws_need = sh.ml_bytes + sh.o_bytes + sh.seq_bytes;
  if (workspace_bytes < ws_need || !workspace)
    return fail(PA_ERR_WORKSPACE, "paged_attn: workspace needs %zu bytes, got %zu", ws_need,
                workspace_bytes);
  if (a->batch == 0) return PA_OK;
  st = validate_attn("paged_attn_fwd", a, sh, workspace, (hipStream_t)stream);
  if (st != PA_OK) return st;
  return launch_attn(a, sh, workspace, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// paged_attn_fwd_noalloc: the same kernels with their workspace in a
// file-scope device array, for callers that cannot allocate
// ---------------------------------------------------------------------------

namespace pa {
namespace {

constexpr size_t kScratchBytes = 32u << 20;  // per GPU, held until the process ends

// The workspace of paged_attn_fwd_noalloc. In host code this name is a host-side
// stand-in, not the device address: only the address from hipGetSymbolAddress
// (kept per device in g_scratch) is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, resolved once per
// device (hipGetSymbolAddress allocates nothing); NULL with an error message
// if it cannot be resolved.
void* scratch_ptr(pa_status* st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = fail(PA_ERR_HIP, "paged_attn_fwd_noalloc: no current HIP device");
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *st = fail(PA_ERR_HIP, "paged_attn_fwd_noalloc: hipGetSymbolAddress: %s",
                 hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *st = PA_OK;
  return p;
}

}  // namespace
}  // namespace pa

extern "C" size_t paged_attn_noalloc_scratch_bytes(void) { return pa::kScratchBytes; }

extern "C" pa_status paged_attn_fwd_noalloc(const pa_attn_args* a, void* stream) {
  Shape sh;
  pa_status st = check_args(a, &sh, true);
  if (st != PA_OK) return st;
  const size_t ws_need = sh.ml_bytes + sh.o_bytes + sh.seq_bytes;
  if (ws_need > kScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "paged_attn_fwd_noalloc: this call needs %zu bytes of workspace, more than the "
                "%zu bytes of the library's scratch array (use paged_attn_fwd)",
                ws_need, kScratchBytes);
  void* ws = scratch_ptr(&st);
  if (st != PA_OK) return st;
  if (a->batch == 0) return PA_OK;
  st = validate_attn("paged_attn_fwd_noalloc", a, sh, ws, (hipStream_t)stream);
  if (st != PA_OK) return st;
  return launch_attn(a, sh, ws, (hipStream_t)stream);
}

extern "C" pa_status pa_plan(const pa_attn_args* a, int32_t* items, int64_t max_items,
                             int32_t* seq_first, int32_t* total, int32_t* info, void* stream) {
  Shape sh;
  pa_status st = check_args(a, &sh, false);
  if (st != PA_OK) return st;
  // at most one item per (sequence, row block, head group, stage)
  const int64_t cap = (int64_t)a->batch * sh.nrb * sh.hgroups *
                      ceil_div(a->max_context_len > 0 ? a->max_context_len : 1, sh.ts);
  if (info) {
    info[0] = sh.nwg;
    info[1] = (int32_t)cap;
    info[2] = sh.ts;
    info[3] = sh.hpu;
    info[4] = sh.run_cost;
    info[5] = sh.nrb;
    info[6] = sh.rpb;
    info[7] = sh.hgroups;
  }
  if (!items) {
    if (!info) return fail(PA_ERR_INVALID_ARG, "pa_plan: items and info both NULL");
    return PA_OK;
  }
  if (max_items < cap) return fail(PA_ERR_WORKSPACE, "pa_plan: needs %lld items", (long long)cap);
  if (!a->block_table || !a->context_lens || !seq_first || !total)
    return fail(PA_ERR_INVALID_ARG, "pa_plan: null pointer");
  if (a->batch == 0) return PA_OK;
  AttnParams p = make_params(a, sh, nullptr);
  p.ws_seq = seq_first;
  hipLaunchKernelGGL(plan_probe_kernel, dim3((unsigned)sh.nwg), dim3(64), 0, (hipStream_t)stream,
                     p, items, cap, total);
  return launch_status("pa_plan kernel");
}

// ---------------------------------------------------------------------------
// selection-driven sparse attention [RELOC] [NULLPAD]
// ---------------------------------------------------------------------------

namespace {

size_t sparse_ws_bytes(const Shape& sh) {
  return sh.ml_bytes + sh.o_bytes + sh.seq_bytes + sh.sp_entries_bytes + sh.sp_masks_bytes +
         sh.sp_vlen_bytes;
}

}  // namespace

extern "C" size_t paged_attn_sparse_workspace_size(const pa_attn_args* a, int32_t topk) {
  Shape sh;
  if (topk < 0 || check_args(a, &sh, false, topk) != PA_OK) return 0;
  return sparse_ws_bytes(sh);
}

extern "C" pa_status paged_attn_sparse(const pa_attn_args* a, const int32_t* sel, int32_t topk,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (topk < 0) return fail(PA_ERR_INVALID_ARG, "paged_attn_sparse: topk < 0");
  Shape sh;
  pa_status st = check_args(a, &sh, true, topk);
  if (st != PA_OK) return st;
  const size_t need = sparse_ws_bytes(sh);
  if (workspace_bytes < need || !workspace)
    return fail(PA_ERR_WORKSPACE, "paged_attn_sparse: workspace needs %zu bytes, got %zu", need,
                workspace_bytes);
  if (a->batch == 0) return PA_OK;
  if (topk > 0 && !sel) return fail(PA_ERR_INVALID_ARG, "paged_attn_sparse: sel is NULL");
  st = validate_attn("paged_attn_sparse", a, sh, workspace, (hipStream_t)stream);
  if (st != PA_OK) return st;
  RingFn fn = pick_ring(a->kv_kind, a->head_dim, sh.nw, sh.RT, q_format(a, sh), kModeSparse);
  if (!fn) return fail(PA_ERR_UNSUPPORTED, "paged_attn_sparse: no kernel for this kind/shape");
  char* base = (char*)workspace + sh.ml_bytes + sh.o_bytes + sh.seq_bytes;
  int32_t* entries = (int32_t*)base;
  uint32_t* masks = (uint32_t*)(base + sh.sp_entries_bytes);
  int32_t* vlen = (int32_t*)(base + sh.sp_entries_bytes + sh.sp_masks_bytes);
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(sparse_plan_kernel, dim3((unsigned)a->batch), dim3(kPlanThreads), 0, s, sel,
                     topk, a->block_table, a->context_lens, a->max_blocks_per_seq,
                     ilog2(a->block_size), a->next_n, sh.sp_cap, entries, masks,
                     (int32_t*)nullptr, vlen);
  st = launch_status("paged_attn_sparse plan kernel");
  if (st != PA_OK) return st;
  AttnParams p = make_params(a, sh, workspace);
  p.context_lens = vlen;  // the merge kernel counts a sequence's items from it
  p.causal = 0;           // the selection alone decides what a row sees
  p.sp_entries = entries;
  p.sp_masks = masks;
  p.sp_cap = sh.sp_cap;
  launch_timed(fn, dim3((unsigned)sh.nwg), dim3(64 * sh.nw), s, p, (const int32_t*)entries,
               (const int32_t*)vlen, (const uint32_t*)masks);
  st = launch_status("paged_attn_sparse ring kernel");
  if (st != PA_OK) return st;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(a->batch * a->num_kv_heads),
                     (unsigned)ceil_div((int64_t)sh.R * a->head_dim / 4, 256)), dim3(256), 0, s,
                     p, a->head_dim);
  return launch_status("paged_attn_sparse merge kernel");
}

extern "C" pa_status pa_sparse_plan(const pa_attn_args* a, const int32_t* sel, int32_t topk,
                                    int32_t* entries, uint32_t* masks, int32_t* count,
                                    int32_t cap, void* stream) {
  if (topk < 0 || cap < 1) return fail(PA_ERR_INVALID_ARG, "pa_sparse_plan: topk < 0 or cap < 1");
  Shape sh;
  pa_status st = check_args(a, &sh, false, topk);
  if (st != PA_OK) return st;
  if (a->batch == 0) return PA_OK;
  if (!entries || !masks || !count || !a->block_table || !a->context_lens || (topk > 0 && !sel))
    return fail(PA_ERR_INVALID_ARG, "pa_sparse_plan: null pointer");
  hipLaunchKernelGGL(sparse_plan_kernel, dim3((unsigned)a->batch), dim3(kPlanThreads), 0,
                     (hipStream_t)stream, sel, topk, a->block_table, a->context_lens,
                     a->max_blocks_per_seq, ilog2(a->block_size), a->next_n, cap, entries, masks,
                     count, (int32_t*)nullptr);
  return launch_status("pa_sparse_plan kernel");
}
