// pa_topk.hip -- top-k token selection over MQA logits on gfx950: the step
// that turns the indexer's per-token logits [FP4API] into the selected token
// ids of each query row that the sparse route consumes [RELOC, Investigation:
// the selected token ids; Upstream check: top-k].
//
// One workgroup of 1024 threads per logits row. Every logit of the row's
// visible tokens is mapped to a 32-bit key that orders like the value (+0
// and -0 alike, NaN below every number). Wave w owns the contiguous token ids
// [c0, c1) of the row. Two routes give the same ids:
//
// Pivot route (rows of up to kTopkLdsKeys tokens). Each wave holds the
// values of its ids in registers (one read of the row, every load in flight
// together). A sample of 4096 keys spread over the row is histogrammed on the
// top 12 key bits; the bins that hold the sample's rank k*S/L -+ (4 sqrt + 16)
// give two key thresholds, and each becomes the smallest value with that key,
// so that value >= threshold tests key >= threshold exactly (NaN and -0
// included). Values above the upper threshold are marked in a per-wave bitmap
// of the ids; values between the two are copied, in id order, to the wave's
// candidate list. If fewer than k values lie above and at least k at or above
// the lower threshold, the k-th largest key T is a candidate: a radix select
// over the candidates alone, one key byte per step (the bytes all candidates
// share are skipped), finds T and how many tokens of key T fit (the lowest ids
// win the ties); the selected candidates join the bitmap, and each wave writes
// the set bits of its ids in order. A row whose sample missed, or whose
// candidates overflow a wave's list, takes the radix route instead.
//
// Radix route. The row's keys are read once into LDS (longer rows re-read the
// logits in every sweep) and the radix select runs over all of them; the
// first digit is 12 bits wide because the logits of one row share few
// sign/exponent bytes (with 8-bit digits about a quarter of a wave's lanes
// would add to the same histogram bin in one atomic). After the first digit
// each wave copies the keys that share it into its own LDS region and counts
// the keys above it; the later digits and the counts of keys above and at T
// look at those candidates only (a wave whose candidates do not fit makes
// every digit sweep all keys). Last, each wave walks its ids in order; prefix
// sums over lanes and over waves -- of tokens of key T and of selected tokens
// -- give every selected token its position: ids come out in ascending order.
#include <type_traits>

#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkLdsKeys = 32768;  // 128 KiB of keys in LDS
constexpr int kTopkDepth = 8;        // 4-key loads in flight per thread while filling it
constexpr int kTopkBins = 4096;      // histogram bins (12-bit digits)
constexpr int kTopkCand = 112;       // candidate keys per wave after the first digit
static_assert(kTopkLdsKeys % (4 * kTopkDepth * kTopkThreads) == 0, "fill rounds");
static_assert(kTopkBins == 4 * kTopkThreads, "four bins per thread in the digit scan");
static_assert(kTopkCand <= 128, "two candidate steps per lane");

struct TopkParams {
  int32_t* sel;
  const void* logits;
  int64_t stride;
  const int32_t* lens;
  int next_n, k;
  int vec;  // rows start 4-element aligned: the fill may load 4 logits at once
};

struct TopkSmem {
  uint32_t keys[kTopkLdsKeys];
  int hist[kTopkBins];
  uint32_t cand_key[kTopkWaves][kTopkCand];
  int32_t cand_id[kTopkWaves][kTopkCand];
  int ws[kTopkWaves];
  int pick[2];  // digit, tokens above it
  int overflow;
};

template <int FMT>
__device__ __forceinline__ float logit_at(const TopkParams& p, int64_t i) {
  if constexpr (FMT == PA_LOGITS_F16)
    return (float)__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(p.logits)[i]);
  else if constexpr (FMT == PA_LOGITS_BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p.logits)[i] << 16);
  else
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

// keys of logits i .. i + 3 (i a multiple of 4 in a row whose start is
// 4-element aligned)
template <int FMT>
__device__ __forceinline__ u4 logit_keys4(const TopkParams& p, int64_t i) {
  u4 k;
  if constexpr (FMT == PA_LOGITS_F32) {
    const f4 v = *reinterpret_cast<const f4*>(static_cast<const float*>(p.logits) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) k[e] = order_key(v[e]);
  } else {
    const u2 v = *reinterpret_cast<const u2*>(static_cast<const uint16_t*>(p.logits) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      k[e] = order_key(FMT == PA_LOGITS_F16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h)
                                            : __uint_as_float(h << 16));
    }
  }
  return k;
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

// Exclusive prefix sum over the waves of a wave-uniform value v.
__device__ __forceinline__ int waves_excl_scan(int v, int* ws) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) ws[wv] = v;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) before += i < wv ? ws[i] : 0;
  __syncthreads();
  return before;
}

__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }
__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }
__device__ __forceinline__ int wave_sum(int x) { return lane_val(wave_incl_scan(x), 63); }

// Selection of one row of L > k tokens. RES: the row's keys are in sm.keys.
template <int FMT, bool RES>
__device__ __forceinline__ void select_row(const TopkParams& p, TopkSmem& sm, int32_t* out,
                                           int64_t base, int L) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int k = p.k;
  const uint64_t below = (1ull << lane) - 1ull;
  // this wave's ids
  const int chunk = (((L + kTopkWaves - 1) / kTopkWaves) + 255) & ~255;
  const int c0 = uni(min(L, wv * chunk)), c1 = uni(min(L, c0 + chunk));

  // keys of ids b .. b + 3 (b = a step's first id + 4 lane); ids at or past
  // c1 are fetched from a valid place and ignored
  auto fetch4 = [&](int b) -> u4 {
    if constexpr (RES) {
      return *reinterpret_cast<const u4*>(&sm.keys[min(b, kTopkLdsKeys - 4)]);
    } else {
      u4 kq;
#pragma unroll
      for (int e = 0; e < 4; ++e) kq[e] = order_key(logit_at<FMT>(p, base + min(b + e, L - 1)));
      return kq;
    }
  };
  // f(keys, first id) for the 4 ids of each lane in every step of the chunk
  auto sweep = [&](auto&& f) {
    for (int b0 = c0; b0 < c1; b0 += 4 * 256) {
      u4 kq[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kq[u] = fetch4(b0 + u * 256 + 4 * lane);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (b0 + u * 256 < c1) f(kq[u], b0 + u * 256 + 4 * lane);
    }
  };

  // ---- radix select of the k-th largest key ----
  uint32_t prefix = 0u, mask = 0u;
  int remaining = k;  // tokens still to take at or below the current prefix
  // one digit: histogram of the keys under the prefix that visit() hands to
  // count(), then the one bin at which the count from the top first reaches
  // `remaining` (thread tid holds bins 4095 - 4 tid - e, e = 0..3)
  auto radix_pass = [&](int shift, uint32_t dmask, auto&& visit) {
    for (int i = tid; i < kTopkBins; i += kTopkThreads) sm.hist[i] = 0;
    __syncthreads();
    visit([&](uint32_t key) {
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1);
    });
    __syncthreads();
    const int4 c4 = *reinterpret_cast<const int4*>(&sm.hist[kTopkBins - 4 - 4 * tid]);
    const int c[4] = {c4.w, c4.z, c4.y, c4.x};
    int total;
    int run = block_excl_scan(c[0] + c[1] + c[2] + c[3], sm.ws, &total);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (run < remaining && run + c[e] >= remaining) {
        sm.pick[0] = kTopkBins - 1 - 4 * tid - e;
        sm.pick[1] = run;
      }
      run += c[e];
    }
    __syncthreads();
    prefix |= (uint32_t)sm.pick[0] << shift;
    mask |= dmask << shift;
    remaining -= sm.pick[1];
    // the next write of pick or hist follows two more barriers
  };
  auto visit_all = [&](auto&& count) {
    sweep([&](u4 kq, int b) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (b + e < c1) count(kq[e]);
    });
  };
  radix_pass(20, 0xFFFu, visit_all);

  // ---- candidates: the keys that share the first digit ----
  const uint32_t d0 = prefix >> 20;
  int n_above = 0, nc = 0;  // per lane: keys above the digit; per wave: candidates
  sweep([&](u4 kq, int b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = b + e < c1;
      const uint32_t top = kq[e] >> 20;
      n_above += ok && top > d0;
      const bool m = ok && top == d0;
      const uint64_t bm = ballot(m);
      const int slot = nc + popc(bm & below);
      if (m && slot < kTopkCand) {
        sm.cand_key[wv][slot] = kq[e];
        sm.cand_id[wv][slot] = b + e;
      }
      nc += popc(bm);
    }
  });
  if (lane == 0 && nc > kTopkCand) sm.overflow = 1;
  n_above = wave_sum(n_above);
  __syncthreads();
  const bool by_cand = sm.overflow == 0;  // workgroup-uniform

  int n_gt = 0, n_eq = 0;  // wave totals of keys above / at T
  if (by_cand) {
    auto visit_cand = [&](auto&& count) {
      for (int i = tid; i < kTopkWaves * kTopkCand; i += kTopkThreads) {
        const int w = i / kTopkCand, j = i - w * kTopkCand;
        if (j < sm.ws[w]) count(sm.cand_key[w][j]);
      }
    };
    // the candidate counts ride in ws between the passes' scans: stored here,
    // read by visit_cand before each pass's scan overwrites ws
    const int ncw = min(nc, kTopkCand);
    auto pass_cand = [&](int shift, uint32_t dmask) {
      if (lane == 0) sm.ws[wv] = ncw;
      __syncthreads();
      radix_pass(shift, dmask, visit_cand);
    };
    pass_cand(8, 0xFFFu);
    pass_cand(0, 0xFFu);
    const uint32_t T = prefix;
    int gt = 0, eq = 0;
    for (int j = lane; j < ncw; j += 64) {
      const uint32_t key = sm.cand_key[wv][j];
      gt += key > T;
      eq += key == T;
    }
    n_gt = n_above + wave_sum(gt);
    n_eq = wave_sum(eq);
  } else {
    radix_pass(8, 0xFFFu, visit_all);
    radix_pass(0, 0xFFu, visit_all);
    const uint32_t T = prefix;
    int gt = 0, eq = 0;
    sweep([&](u4 kq, int b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = b + e < c1;
        gt += ok && kq[e] > T;
        eq += ok && kq[e] == T;
      }
    });
    n_gt = wave_sum(gt);
    n_eq = wave_sum(eq);
  }
  const uint32_t T = prefix;

  // ---- positions ----
  const int eq_before = waves_excl_scan(n_eq, sm.ws);
  // tokens of key T are taken lowest id first: `remaining` of them
  const int eq_take = max(0, min(n_eq, remaining - eq_before));
  int pos = waves_excl_scan(n_gt + eq_take, sm.ws), eq_seen = 0;
  sweep([&](u4 kq, int b) {
    bool gt[4], eq[4];
    int ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = b + e < c1;
      gt[e] = ok && kq[e] > T;
      eq[e] = ok && kq[e] == T;
      ne += eq[e];
    }
    const int eq_incl = wave_incl_scan(ne);
    int rank = eq_seen + eq_incl - ne;  // tokens of key T before this lane's first id
    bool take[4];
    int nt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      take[e] = gt[e] || (eq[e] && rank < eq_take);
      rank += eq[e];
      nt += take[e];
    }
    const int take_incl = wave_incl_scan(nt);
    int q = pos + take_incl - nt;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (take[e]) out[q++] = b + e;
    pos += lane_val(take_incl, 63);
    eq_seen += lane_val(eq_incl, 63);
  });
}

// ---------------------------------------------------------------------------
// pivot route
// ---------------------------------------------------------------------------

constexpr int kPivSteps = kTopkLdsKeys / (kTopkWaves * 256);  // 256-id steps per wave
constexpr int kPivSamples = 4;                               // sampled keys per thread
constexpr int kPivCand = 480;                                // candidates per wave
static_assert(kPivSteps % 2 == 0 && kPivSteps >= 2 * kPivSamples, "sample placement");

struct PivotSmem {
  int hist[kTopkBins];      // sample histogram on the top 12 key bits
  int dhist[4][256];        // candidate histograms, one per 8-bit digit
  uint32_t cand_val[kTopkWaves][kPivCand];  // fp32 bits of the candidates' values
  int32_t cand_id[kTopkWaves][kPivCand];
  uint32_t bits[kTopkWaves][kPivSteps * 8];  // bit i: id c0 + i of the wave is selected
  int ws[2][kTopkWaves];                     // alternate buffers of the block scans
  int tot[3][kTopkWaves];                    // per wave: keys above, candidates, overflow
  int cnt[2][kTopkWaves];                    // per wave: candidates above T, at T
  int nsamp;
  int piv[2];  // d_hi, d_lo
};

// OR of x over each group of 8 lanes (lanes 8g .. 8g + 7), in every lane of
// the group: quad_perm swaps of neighbours and of pairs, then the mirror of
// the half-row.
__device__ __forceinline__ uint32_t or8(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false); // row_half_mirror
  return x;
}

// set bits of m in the lanes below this one
__device__ __forceinline__ int count_below(uint64_t m, int acc) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)acc));
}

// Exclusive prefix sum over the workgroup with one barrier: `ws` alternates
// between two buffers (*flip), so a buffer is rewritten only after the
// barrier of the next scan, which follows every read of it.
__device__ __forceinline__ int block_excl_scan1(int x, int (*ws)[kTopkWaves], int* flip) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int* b = ws[*flip];
  *flip ^= 1;
  const int incl = wave_incl_scan(x);
  if (lane == 63) b[wv] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) before += i < wv ? b[i] : 0;
  return before + incl - x;
}

// The smallest value whose key is at least K (K > 0): value >= it exactly
// when key(value) >= K, for every value including -0 and infinities (NaN is
// never >= it, and its key 0 is below K). Keys 1 .. 0x7FFFFE belong to no
// value (they would be negative NaNs), so those K act as 0x7FFFFF = key(-inf).
__device__ __forceinline__ float key_floor_value(uint32_t K) {
  if (K & 0x80000000u) return __uint_as_float(K & 0x7FFFFFFFu);
  if (K <= 0x007FFFFFu) return -__builtin_inff();
  return __uint_as_float(~K);
}

// Values of the wave's ids into registers: step u, lane l holds ids
// c0 + 256 u + 4 l + e. Reads stay inside the row's first L ids or, with
// 4-aligned rows, inside the aligned group of 4 that holds id L - 1; every
// load is issued before the first is used.
template <int FMT>
__device__ __forceinline__ void load_row_vals(const TopkParams& p, int64_t base, int c0, int L,
                                              f4 (&v)[kPivSteps]) {
  const int lane = threadIdx.x & 63;
  if (p.vec) {
    const int qlast = (L - 1) >> 2;
    if constexpr (FMT == PA_LOGITS_F32) {
#pragma unroll
      for (int u = 0; u < kPivSteps; ++u) {
        const int q = min((c0 >> 2) + 64 * u + lane, qlast);
        v[u] = *reinterpret_cast<const f4*>(static_cast<const float*>(p.logits) + base + 4 * (int64_t)q);
      }
    } else {
      u2 raw[kPivSteps];
#pragma unroll
      for (int u = 0; u < kPivSteps; ++u) {
        const int q = min((c0 >> 2) + 64 * u + lane, qlast);
        raw[u] = *reinterpret_cast<const u2*>(static_cast<const uint16_t*>(p.logits) + base + 4 * (int64_t)q);
      }
#pragma unroll
      for (int u = 0; u < kPivSteps; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h = (raw[u][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          v[u][e] = FMT == PA_LOGITS_F16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h)
                                         : __uint_as_float(h << 16);
        }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPivSteps; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[u][e] = logit_at<FMT>(p, base + min(c0 + 256 * u + 4 * lane + e, L - 1));
  }
}

// Returns false (workgroup-uniform, nothing written to out) when the pivots
// missed T or the candidates overflowed.
template <int FMT>
__device__ __forceinline__ bool select_pivot(const TopkParams& p, PivotSmem& sm, int32_t* out,
                                             int64_t base, int L) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int k = p.k;
  const uint64_t below = (1ull << lane) - 1ull;
  const int chunk = (((L + kTopkWaves - 1) / kTopkWaves) + 255) & ~255;  // <= 256 kPivSteps
  const int c0 = uni(min(L, wv * chunk)), c1 = uni(min(L, c0 + chunk));
  int flip = 0;

  f4 v[kPivSteps];
  load_row_vals<FMT>(p, base, c0, L, v);
  // histograms cleared while the loads are in flight
  *reinterpret_cast<int4*>(&sm.hist[4 * tid]) = int4{0, 0, 0, 0};
  (&sm.dhist[0][0])[tid] = 0;
  if (tid == 0) {
    sm.nsamp = 0;
    sm.piv[0] = kTopkBins - 1;
    sm.piv[1] = 0;
  }
  __syncthreads();

  // ---- sample histogram: keys of steps 2j + (l & 1), slot (l >> 4) & 3 ----
  {
    // the picks are mask arithmetic, not selects: a select between array
    // elements becomes a dynamic index, and the array would leave registers
    const int e = (lane >> 4) & 3;
    const uint32_t om = 0u - (uint32_t)(lane & 1);
    uint32_t em[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) em[c] = 0u - (uint32_t)(e == c);
    int nv = 0;
#pragma unroll
    for (int j = 0; j < kPivSamples; ++j) {
      uint32_t x = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t x0 = __float_as_uint(v[2 * j][c]), x1 = __float_as_uint(v[2 * j + 1][c]);
        x |= (x0 ^ ((x0 ^ x1) & om)) & em[c];
      }
      const bool ok = c0 + 256 * (2 * j + (lane & 1)) + 4 * lane + e < c1;
      if (ok) atomicAdd(&sm.hist[order_key(__uint_as_float(x)) >> 20], 1);
      nv += popc(ballot(ok));
    }
    if (lane == 0) atomicAdd(&sm.nsamp, nv);
  }
  __syncthreads();
  {
    const int S = sm.nsamp;
    const float sr = (float)k * (float)S / (float)L;  // expected sample count at or above T
    const float mg = 4.f * sqrtf(sr) + 16.f;
    const int r_hi = (int)floorf(sr - mg), r_lo = (int)ceilf(sr + mg);
    // thread tid holds bins 4095 - 4 tid - e (descending); the pivot bins hold
    // the sample ranks r_hi and r_lo (0 = the largest sampled key)
    const int4 c4 = *reinterpret_cast<const int4*>(&sm.hist[kTopkBins - 4 - 4 * tid]);
    const int c[4] = {c4.w, c4.z, c4.y, c4.x};
    int run = block_excl_scan1(c[0] + c[1] + c[2] + c[3], sm.ws, &flip);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = kTopkBins - 1 - 4 * tid - e;
      if (run <= r_hi && r_hi < run + c[e]) sm.piv[0] = d;
      if (run <= r_lo && r_lo < run + c[e]) sm.piv[1] = d;
      run += c[e];
    }
  }
  __syncthreads();
  const uint32_t d_hi = (uint32_t)sm.piv[0], d_lo = (uint32_t)sm.piv[1];
  // above: key >= (d_hi + 1) << 20; candidate: not above and key >= d_lo << 20.
  // With no keys above, f_hi is NaN (nothing is >= it); with d_lo = 0 every
  // value not above is a candidate, NaN included (its key 0 is >= 0).
  const bool lo_all = d_lo == 0;
  const float f_hi = d_hi < kTopkBins - 1 ? key_floor_value((d_hi + 1) << 20)
                                          : __builtin_nanf("");
  const float f_lo = lo_all ? -__builtin_inff() : key_floor_value(d_lo << 20);

  // ---- classify: above -> bitmap; candidates -> the wave's list, in id order ----
  int na = 0, nc = 0;  // per wave: values above, candidates
  bool ovf_w = false;
  // one step of 256 ids; FULL: all of them below c1 (no per-id bound test);
  // LOALL: d_lo = 0
  auto step = [&](auto full_c, auto loall_c, int u) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value, LOALL = decltype(loall_c)::value;
    const int b = c0 + 256 * u + 4 * lane;
    uint32_t nib = 0;
    bool cf[4];
    uint64_t cm[4];
    int nb = nc;  // candidates before this lane's first id
    int ns = 0;   // candidates in this step
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = v[u][e];
      bool a = x >= f_hi;
      bool g = LOALL ? !(x < f_lo) : x >= f_lo;
      if constexpr (!FULL) {
        const bool ok = b + e < c1;
        a = a && ok;
        g = g && ok;
      }
      cf[e] = g && !a;
      na += popc(ballot(a));
      cm[e] = ballot(cf[e]);
      ns += popc(cm[e]);
      nib |= a ? 1u << e : 0u;
      nb = count_below(cm[e], nb);
    }
    const uint32_t word = or8(nib << (4 * (lane & 7)));
    if ((lane & 7) == 0) sm.bits[wv][8 * u + (lane >> 3)] = word;
    if (nc + ns <= kPivCand) {  // wave-uniform; past it the row takes the radix route
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cf[e]) {
          sm.cand_val[wv][nb] = __float_as_uint(v[u][e]);
          sm.cand_id[wv][nb] = b + e;
        }
        nb += cf[e];
      }
    } else {
      ovf_w = true;
    }
    nc += ns;
  };
  auto classify = [&](auto loall_c) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPivSteps; ++u) {
      if (c0 + 256 * u >= c1) continue;  // wave-uniform
      if (c0 + 256 * (u + 1) <= c1)
        step(std::true_type{}, loall_c, u);
      else
        step(std::false_type{}, loall_c, u);
    }
  };
  if (lo_all)
    classify(std::true_type{});
  else
    classify(std::false_type{});
  if (lane == 0) {
    sm.tot[0][wv] = na;
    sm.tot[1][wv] = min(nc, kPivCand);
    sm.tot[2][wv] = ovf_w;
  }
  __syncthreads();
  int A = 0, C = 0, ovf = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    A += sm.tot[0][i];
    C += sm.tot[1][i];
    ovf |= sm.tot[2][i];
  }
  if (ovf || A >= k || A + C < k) return false;

  // ---- radix select among the candidates: the (k - A)-th largest ----
  // Candidate keys lie in [d_lo << 20, d_hi << 20 | 0xFFFFF]; their common
  // leading bytes are known. Each remaining byte: one histogram, one barrier,
  // and every wave finds the same digit from the 256 bins (the phases from
  // here on are chains of dependent LDS steps: spread over all waves, each
  // wave's chain stays short).
  const int nc_w = sm.tot[1][wv];  // this wave's candidates
  uint32_t prefix = 0u, mask = 0u;
  int remaining = k - A;
  const uint32_t klo = d_lo << 20, khi = (d_hi << 20) | 0xFFFFFu;
  int first = 0;
  while (first < 4 && ((klo ^ khi) >> (24 - 8 * first)) == 0u) {
    mask |= 255u << (24 - 8 * first);
    ++first;
  }
  prefix = klo & mask;
#pragma unroll 1
  for (int pass = first; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    int* dh = sm.dhist[pass];
    for (int j0 = 0; j0 < nc_w; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t key = j < nc_w ? order_key(__uint_as_float(sm.cand_val[wv][j])) : 0u;
      const bool act = j < nc_w && (key & mask) == prefix;
      const int d = (int)((key >> shift) & 255u);
      // most candidates share the digit of the first active lane: one add for them
      const uint64_t am = ballot(act);
      if (am) {
        const int fl = __builtin_ctzll(am);
        const int ld = __builtin_amdgcn_readlane(d, fl);
        const uint64_t same = ballot(act && d == ld);
        if (lane == fl) atomicAdd(&dh[ld], popc(same));
        if (act && d != ld) atomicAdd(&dh[d], 1);
      }
    }
    __syncthreads();
    // lane l holds digits 255 - 4 l - e (descending)
    const int4 c4 = *reinterpret_cast<const int4*>(&dh[252 - 4 * lane]);
    const int c[4] = {c4.w, c4.z, c4.y, c4.x};
    const int sum = c[0] + c[1] + c[2] + c[3];
    int run = wave_incl_scan(sum) - sum, hd = -1, hr = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (run < remaining && run + c[e] >= remaining) {
        hd = 255 - 4 * lane - e;
        hr = run;
      }
      run += c[e];
    }
    const int hl = __builtin_ctzll(ballot(hd >= 0));
    prefix |= (uint32_t)__builtin_amdgcn_readlane(hd, hl) << shift;
    mask |= 255u << shift;
    remaining -= __builtin_amdgcn_readlane(hr, hl);
  }
  const uint32_t T = prefix;  // `remaining` tokens of key T are taken, lowest ids first

  // ---- per wave: candidates above and at T; then positions ----
  int gt = 0, eq = 0;
  for (int j = lane; j < nc_w; j += 64) {
    const uint32_t key = order_key(__uint_as_float(sm.cand_val[wv][j]));
    gt += key > T;
    eq += key == T;
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (lane == 0) {
    sm.cnt[0][wv] = gt;
    sm.cnt[1][wv] = eq;
  }
  __syncthreads();
  int eq_before = 0, pos = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    if (i < wv) {
      const int ne = sm.cnt[1][i];
      pos += sm.tot[0][i] + sm.cnt[0][i] + max(0, min(ne, remaining - eq_before));
      eq_before += ne;
    }
  }
  // selected candidates join the bitmap
  int seen = eq_before;
  for (int j0 = 0; j0 < nc_w; j0 += 64) {
    const int j = j0 + lane;
    const bool ok = j < nc_w;
    const uint32_t key = ok ? order_key(__uint_as_float(sm.cand_val[wv][j])) : 0u;
    const int id = ok ? sm.cand_id[wv][j] : c0;
    const bool at = ok && key == T;
    const uint64_t me = ballot(at);
    const bool sel = ok && (key > T || (at && count_below(me, seen) < remaining));
    if (sel) atomicOr(&sm.bits[wv][(id - c0) >> 5], 1u << ((id - c0) & 31));
    seen += popc(me);
  }

  // ---- output: the set bits of each wave's ids, in order ----
  const int nwords = (c1 - c0 + 31) >> 5;
  uint32_t word = lane < nwords ? sm.bits[wv][lane] : 0u;
  const int cnt = __builtin_popcount(word);
  pos += wave_incl_scan(cnt) - cnt;
  while (word) {  // (the set bits number k; the bound only keeps writes inside the row)
    if (pos < k) out[pos] = c0 + 32 * lane + __builtin_ctz(word);
    ++pos;
    word &= word - 1u;
  }
  return true;
}

template <int FMT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) union {
    TopkSmem radix;
    PivotSmem pivot;
  } smu;
  TopkSmem& sm = smu.radix;
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
  if (L <= kTopkLdsKeys) {
    if (select_pivot<FMT>(p, smu.pivot, out, base, L)) return;
    __syncthreads();  // the radix route reuses the pivot route's LDS
  }
  if (tid == 0) sm.overflow = 0;
  if (L > kTopkLdsKeys) {
    __syncthreads();
    select_row<FMT, false>(p, sm, out, base, L);
    return;
  }
  // keys of the row in LDS: loads read a clamped (valid) place so that none
  // waits behind a branch, and only ids below L are stored
  if (p.vec) {
    const int nq = L >> 2;  // whole groups of 4
    for (int g0 = 0; g0 < nq; g0 += kTopkDepth * kTopkThreads) {
      u4 kq[kTopkDepth];
#pragma unroll
      for (int u = 0; u < kTopkDepth; ++u)
        kq[u] = logit_keys4<FMT>(p, base + 4 * (int64_t)min(g0 + u * kTopkThreads + tid, nq - 1));
#pragma unroll
      for (int u = 0; u < kTopkDepth; ++u) {
        const int g = g0 + u * kTopkThreads + tid;
        if (g < nq) *reinterpret_cast<u4*>(&sm.keys[4 * g]) = kq[u];
      }
    }
    const int t = 4 * nq + tid;
    if (t < L) sm.keys[t] = order_key(logit_at<FMT>(p, base + t));
  } else {
    for (int t0 = 0; t0 < L; t0 += 4 * kTopkDepth * kTopkThreads) {
      float v[4 * kTopkDepth];
#pragma unroll
      for (int u = 0; u < 4 * kTopkDepth; ++u)
        v[u] = logit_at<FMT>(p, base + min(t0 + u * kTopkThreads + tid, L - 1));
#pragma unroll
      for (int u = 0; u < 4 * kTopkDepth; ++u) {
        const int t = t0 + u * kTopkThreads + tid;
        if (t < L) sm.keys[t] = order_key(v[u]);
      }
    }
  }
  __syncthreads();
  select_row<FMT, true>(p, sm, out, base, L);
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
  p.next_n = a->next_n;
  p.k = a->k;
  const size_t esz = a->logits_format == PA_LOGITS_F32 ? 4 : 2;
  p.vec = a->logits_row_stride % 4 == 0 && (uintptr_t)a->logits % (4 * esz) == 0;
  const dim3 grid((unsigned)rows), block(kTopkThreads);
  if (a->logits_format == PA_LOGITS_F16)
    launch_timed(topk_kernel<PA_LOGITS_F16>, grid, block, (hipStream_t)stream, p);
  else if (a->logits_format == PA_LOGITS_BF16)
    launch_timed(topk_kernel<PA_LOGITS_BF16>, grid, block, (hipStream_t)stream, p);
  else
    launch_timed(topk_kernel<PA_LOGITS_F32>, grid, block, (hipStream_t)stream, p);
  return launch_status("pa_topk_select kernel");
}
