/*
 * oracle.c -- plain CPU reference for paged attention over a quantized,
 * block-table-indexed KV cache, the MXFP4 paged MQA logits, and the KV insert.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library shares no code,
 * header, table or helper with it, and neither links the other.
 *
 * It is deliberately slow and literal: every value is decoded from its bit
 * fields by the format's definition, every token is looked up through the
 * block table one at a time, and sums run in ascending index order.
 *
 * Precision. A dequantized cache value is fp32(code) * fp32(scale), one fp32
 * rounding, which is what the per-channel scale page ("Normalize the
 * PER_CHANNEL K scale folded into Q for paged XQA", Description) calls the
 * portable FP32 product. Attention sums (q.k, the softmax denominator and the
 * weighted sum of V) are accumulated in double, so the reference error is far
 * below the fp16 output tolerance. The MQA logits follow the fp32 contract of
 * the fp4_paged_mqa_logits API page (float32 weights and output): per-head
 * dot products in fp32, then an fmaf chain over heads in ascending order.
 *
 * Sources (each function cites the passage it follows):
 *  [P1] "Stop grouped-page4 null-block padding from leaking E4M3 NaN"
 *  [P2] "Normalize the PER_CHANNEL K scale folded into Q for paged XQA"
 *  [P4] "DeepSeek-V4.1 Q pad + fused KV insert" (the KV-only insert path)
 *  [P5] "flashinfer.fp4_paged_mqa_logits" API documentation
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_KV_F16 0
#define ORC_KV_BF16 1
#define ORC_KV_E4M3 2
#define ORC_KV_INT8 3
#define ORC_KV_INT4 4

#define ORC_SCALE_NONE 0
#define ORC_SCALE_PER_TENSOR 1
#define ORC_SCALE_PER_CHANNEL 2

/* ------------------------------------------------------------------ */
/* Scalar codecs                                                       */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float orc_f16_to_f32(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + f, e - 25);
  return (float)(s ? -v : v);
}

/* bfloat16 is the upper half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double to binary16, round-to-nearest-even, overflow to infinity. */
uint16_t orc_f64_to_f16(double x) {
  if (isnan(x)) return 0x7E00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);          /* a lies in [2^(e2-1), 2^e2) */
  int lead = e2 - 1;
  if (lead < -14) lead = -14; /* subnormal range: spacing 2^-24 */
  double quantum = ldexp(1.0, lead - 10);
  double r = nearbyint(a / quantum) * quantum; /* default rounding mode: ties to even */
  if (r > 65504.0) return sign | 0x7C00;
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
  int er;
  frexp(r, &er);
  int exp_field = er - 1 + 15;
  double frac = r / ldexp(1.0, er - 1) - 1.0; /* in [0, 1) */
  return sign | (uint16_t)(exp_field << 10) | (uint16_t)(frac * 1024.0);
}

/* Round a float to bfloat16, round-to-nearest-even (NaN kept quiet). */
uint16_t orc_f32_to_bf16(float x) {
  if (isnan(x)) return 0x7FC0;
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t keep = u >> 16, rest = u & 0xFFFF;
  if (rest > 0x8000 || (rest == 0x8000 && (keep & 1))) keep += 1;
  return (uint16_t)keep;
}

/* OCP FP8 E4M3 ("FN"): 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinity; 0x7F and 0xFF are NaN [P1, Root cause: NaN bytes 0x7F/0xFF];
 * largest finite magnitude 448 (code 0x7E). */
float orc_e4m3_to_f32(uint8_t c) {
  int s = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexpf((float)m, -9); /* (m/8) * 2^-6 */
  else
    v = ldexpf(8.0f + (float)m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* Nearest E4M3 code, ties to the even code, saturating to +-448; NaN -> 0x7F.
 * Found by scanning all finite non-negative codes: slow and obviously right. */
uint8_t orc_f32_to_e4m3(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int best = 0;
  double bestd = a;
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs((double)orc_e4m3_to_f32((uint8_t)c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return sign | (uint8_t)best;
}

/* Signed INT8 and INT4 codes: symmetric round-to-nearest-even with clamps
 * +-127 and +-7, the "/127" and "/7" scale ranges of [P2, Description]. */
int orc_round_clamp(float y, int lim) {
  if (isnan(y)) return 0;
  float r = nearbyintf(y);
  if (r > (float)lim) r = (float)lim;
  if (r < (float)-lim) r = (float)-lim;
  return (int)r;
}

/* INT4 nibble (two's complement, 4 bits) -> integer in [-8, 7]. */
int orc_int4_value(int nib) { return nib >= 8 ? nib - 16 : nib; }

/* OCP E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit. */
float orc_e2m1_to_f32(uint8_t nib) {
  int s = (nib >> 3) & 1;
  int e = (nib >> 1) & 3;
  int m = nib & 1;
  float v = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
  return s ? -v : v;
}

/* OCP UE8M0 scale factor: 2^(e - 127); 0xFF is NaN. */
float orc_ue8m0_to_f32(uint8_t e) {
  if (e == 0xFF) return NAN;
  return ldexpf(1.0f, (int)e - 127);
}

/*
 * E2M1 code of y, round to nearest with ties to the even code, saturating to
 * +-6 (the largest E2M1 magnitude). The magnitude code is the index of the
 * nearest of the 8 representable magnitudes; the sign bit is y's sign bit.
 * (Reading: the pages give no rounding rule for FP4 writes; nearest-even with
 * saturation is the OCP Microscaling conversion.)
 */
uint8_t orc_f32_to_e2m1(float y) {
  float a = fabsf(y);
  int best = 0;
  float bestd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    float d = fabsf(a - orc_e2m1_to_f32((uint8_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      bestd = d;
      best = c;
    }
  }
  if (a > 6.0f) best = 7; /* saturate: ties above 6 cannot occur, 6 is the top code */
  return (uint8_t)(best | (signbit(y) ? 8 : 0));
}

/*
 * UE8M0 scale byte of a 32-value group with largest magnitude amax (OCP
 * Microscaling rule, a reading: the pages print no quantizer): the shared
 * scale is 2^(floor(log2(amax)) - 2), 2 being the exponent of E2M1's largest
 * power of two, clamped to the finite bytes [0, 254]; an all-zero group gets
 * byte 0.
 */
uint8_t orc_mx_scale_byte(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  frexpf(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1 */
  int b = (e - 1) - 2 + 127;
  return (uint8_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

/* ------------------------------------------------------------------ */
/* Paged KV element access                                             */
/* ------------------------------------------------------------------ */

static int elem_bits(int kind) {
  if (kind == ORC_KV_F16 || kind == ORC_KV_BF16) return 16;
  if (kind == ORC_KV_INT4) return 4;
  return 8;
}

/* Code value of element (slot, head, d) of physical block blk, as a float.
 * The cache is [num_blocks, block_size, kv_heads, head_dim] [P5, kv_fused /
 * block_table parameters]; INT4 keeps element 2j in the low nibble. */
static float cache_code(const uint8_t* cache, int kind, int64_t blk, int slot, int hk, int d,
                        int bs, int Hkv, int D) {
  int64_t row = (blk * bs + slot) * Hkv + hk;
  int64_t row_bytes = (int64_t)D * elem_bits(kind) / 8;
  const uint8_t* p = cache + row * row_bytes;
  if (kind == ORC_KV_F16) {
    uint16_t h;
    memcpy(&h, p + 2 * d, 2);
    return orc_f16_to_f32(h);
  }
  if (kind == ORC_KV_BF16) {
    uint16_t h;
    memcpy(&h, p + 2 * d, 2);
    return orc_bf16_to_f32(h);
  }
  if (kind == ORC_KV_E4M3) return orc_e4m3_to_f32(p[d]);
  if (kind == ORC_KV_INT8) return (float)(int8_t)p[d];
  {
    uint8_t byte = p[d / 2];
    int nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
    return (float)orc_int4_value(nib);
  }
}

static float scale_of(const float* scale, int mode, int hk, int d, int D) {
  if (mode == ORC_SCALE_PER_TENSOR) return scale[0];
  if (mode == ORC_SCALE_PER_CHANNEL) return scale[hk * D + d];
  return 1.0f;
}

/* Dequantized value: fp32(code) * fp32(scale), one rounding [P2, Description:
 * the portable kernel keeps the q*k_scale product in FP32]. */
static float deq(const uint8_t* cache, int kind, const float* scale, int mode, int64_t blk,
                 int slot, int hk, int d, int bs, int Hkv, int D) {
  return cache_code(cache, kind, blk, slot, hk, d, bs, Hkv, D) * scale_of(scale, mode, hk, d, D);
}

/* Element-wise decode of a flat code array (the dequantization probe):
 * element i uses scale[i % channels] per channel, scale[0] per tensor. */
void orc_dequantize(int kind, const uint8_t* codes, int64_t n, const float* scale, int mode,
                    int64_t channels, float* out) {
  for (int64_t i = 0; i < n; ++i) {
    float code;
    if (kind == ORC_KV_E4M3)
      code = orc_e4m3_to_f32(codes[i]);
    else if (kind == ORC_KV_INT8)
      code = (float)(int8_t)codes[i];
    else if (kind == ORC_KV_INT4) {
      uint8_t byte = codes[i / 2];
      code = (float)orc_int4_value((i % 2 == 0) ? (byte & 15) : (byte >> 4));
    } else {
      uint16_t h;
      memcpy(&h, codes + 2 * i, 2);
      code = (kind == ORC_KV_F16) ? orc_f16_to_f32(h) : orc_bf16_to_f32(h);
    }
    float s = 1.0f;
    if (mode == ORC_SCALE_PER_TENSOR) s = scale[0];
    if (mode == ORC_SCALE_PER_CHANNEL) s = scale[i % channels];
    out[i] = code * s;
  }
}

/* ------------------------------------------------------------------ */
/* Threads                                                             */
/* ------------------------------------------------------------------ */

/* The attention and logits loops run their independent units (a sequence and
 * KV head, or a logits row) on OpenMP threads; every sum inside a unit keeps
 * its stated order, so the result does not depend on the thread count.
 * n > 0 sets the thread count, n <= 0 restores one thread per processor. */
void orc_set_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
#else
  (void)n;
#endif
}

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Paged attention                                                     */
/* ------------------------------------------------------------------ */

/* Query value: fp16 or bf16 bits. */
static float q_value(const uint16_t* q, int q_is_bf16, int64_t idx) {
  return q_is_bf16 ? orc_bf16_to_f32(q[idx]) : orc_f16_to_f32(q[idx]);
}

/* Dequantized K and V rows of tokens t < L of sequence b for KV head hk (only
 * tokens with want[t] != 0 when want is given): kd[t * D + d], vd[t * D + d].
 * csum[t] = sum over d of |K code|. A token mapped outside the real blocks
 * (block 0 is the null block) is a harness error: returns -1. */
static int gather_rows(float* kd, float* vd, double* csum, const unsigned char* want,
                       const uint8_t* k_cache, const uint8_t* v_cache, int kind,
                       const float* k_scale, int k_mode, const float* v_scale, int v_mode,
                       const int32_t* table_row, int L, int hk, int bs, int Hkv, int D,
                       int64_t num_blocks) {
  for (int t = 0; t < L; ++t) {
    if (want && !want[t]) continue;
    int64_t blk = table_row[t / bs];
    if (blk <= 0 || blk >= num_blocks) return -1;
    double c = 0.0;
    for (int d = 0; d < D; ++d) {
      float kc = cache_code(k_cache, kind, blk, t % bs, hk, d, bs, Hkv, D);
      kd[(int64_t)t * D + d] = kc * scale_of(k_scale, k_mode, hk, d, D); /* = deq() */
      vd[(int64_t)t * D + d] = deq(v_cache, kind, v_scale, v_mode, blk, t % bs, hk, d, bs, Hkv, D);
      c += fabs((double)kc);
    }
    csum[t] = c;
  }
  return 0;
}

/*
 * One query row over its visible tokens (vis[t] != 0, t < L): scores
 * s_t = softmax_scale * sum over d ascending of q[d] * K_t[d] (double), then
 * softmax and the weighted sum of V, both over t ascending; the row is +0
 * when no token is visible.
 *
 * Conditioning (cond != NULL): cond[0] = s_top1 - s_top2 (the fp64 gap
 * between the two largest scores, +inf with fewer than two tokens), cond[1] =
 * eps, a bound on the error of one score computed with fp32 accumulation:
 * eps = max over t of softmax_scale * ((D + 8) * 2^-24 * sum_d |q[d] K_t[d]|
 * + fold * 2^-25 * kmax * csum[t]), where the second term (folded per-channel
 * K scales, kmax = max|k_scale|) bounds a 2^-25 absolute error per element of
 * a q * k_scale / kmax split into two fp16 parts. cond[2] = the number of
 * tokens with s_t >= s_top1 - 8 eps - 32, the tokens whose softmax weight can
 * exceed e^-32 of the largest under such errors; vlo[d] / vhi[d] = min / max
 * of V_t[d] over them; vsens[d] = sum_t p_t |V_t[d] - out[d]| / l, the
 * first-order change of out[d] per unit of score error common to no token
 * (|d out / d s| summed over t).
 */
static void attend_row(double* orow, const float* qf, const float* kd, const float* vd,
                       const double* csum, const unsigned char* vis, int L, int D,
                       float softmax_scale, double* s, double* ab, double* cond, double* vlo,
                       double* vhi, double* vsens, double fold_kmax) {
  for (int d = 0; d < D; ++d) orow[d] = 0.0;
  double m = -INFINITY;
  int n = 0;
  for (int t = 0; t < L; ++t) {
    if (!vis[t]) continue;
    double acc = 0.0, aabs = 0.0;
    for (int d = 0; d < D; ++d) {
      double x = (double)qf[d] * (double)kd[(int64_t)t * D + d];
      acc += x;
      aabs += fabs(x);
    }
    s[t] = (double)softmax_scale * acc;
    ab[t] = (double)softmax_scale * ((D + 8) * ldexp(1.0, -24) * aabs +
                                     ldexp(1.0, -25) * fold_kmax * csum[t]);
    if (s[t] > m) m = s[t];
    ++n;
  }
  if (cond) {
    double second = -INFINITY, eps = 0.0;
    int top = 0;
    for (int t = 0; t < L; ++t) {
      if (!vis[t]) continue;
      if (ab[t] > eps) eps = ab[t];
      if (s[t] == m && !top) {
        top = 1;
        continue;
      }
      if (s[t] > second) second = s[t];
    }
    cond[0] = n >= 2 ? m - second : INFINITY;
    cond[1] = eps;
    cond[2] = 0.0;
    for (int d = 0; d < D; ++d) {
      vlo[d] = INFINITY;
      vhi[d] = -INFINITY;
    }
    for (int t = 0; t < L; ++t) {
      if (!vis[t] || s[t] < m - 8.0 * eps - 32.0) continue;
      cond[2] += 1.0;
      for (int d = 0; d < D; ++d) {
        double v = vd[(int64_t)t * D + d];
        if (v < vlo[d]) vlo[d] = v;
        if (v > vhi[d]) vhi[d] = v;
      }
    }
  }
  if (vsens)
    for (int d = 0; d < D; ++d) vsens[d] = 0.0;
  if (n == 0) return;
  double l = 0.0;
  for (int t = 0; t < L; ++t) {
    if (!vis[t]) continue;
    s[t] = exp(s[t] - m);
    l += s[t];
  }
  for (int t = 0; t < L; ++t) {
    if (!vis[t]) continue;
    for (int d = 0; d < D; ++d) orow[d] += s[t] * (double)vd[(int64_t)t * D + d];
  }
  for (int d = 0; d < D; ++d) orow[d] /= l;
  if (vsens) {
    for (int t = 0; t < L; ++t) {
      if (!vis[t]) continue;
      for (int d = 0; d < D; ++d) vsens[d] += s[t] * fabs((double)vd[(int64_t)t * D + d] - orow[d]);
    }
    for (int d = 0; d < D; ++d) vsens[d] /= l;
  }
}

static float max_abs(const float* x, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; ++i)
    if (fabsf(x[i]) > m) m = fabsf(x[i]);
  return m;
}

/*
 * out[b, i, h, :] = softmax(softmax_scale * q[b,i,h,:] . K_t) @ V_t over the
 * visible tokens t of sequence b, dequantize first [P2, Description: portable
 * path], read through block_table [P5, block_table parameter].
 *
 * Readings where the pages are silent:
 *  - q and out are [B, next_n, Hq, D]; query head h reads KV head
 *    h / (Hq / Hkv) (contiguous groups). q is fp16, or bf16 with q_is_bf16.
 *  - Query row i sits at absolute position L_b - next_n + i; with causal set
 *    it sees tokens t <= that position, otherwise all t < L_b.
 *  - No visible token: the output row is +0.
 *  - Tokens past L_b are never read, so the null block (physical block 0
 *    [P1, Root cause]) and tail slots cannot influence the result. A token
 *    t < L_b mapped to block 0 is a harness error (returns -1).
 *
 * Scores, softmax and the weighted sum are accumulated in double; `out` is
 * the double result (the caller rounds to its output dtype). cond / vrange
 * (NULL to skip): per output row (b, i, h) the conditioning of attend_row,
 * cond[row * 4 + {0, 1, 2}], vrange[(row * 3 + {0, 1, 2}) * D + d] = vlo, vhi,
 * vsens.
 */
int orc_paged_attn(double* out, const uint16_t* q, int q_is_bf16, const uint8_t* k_cache,
                   const uint8_t* v_cache, int kv_kind, const float* k_scale, int k_scale_mode,
                   const float* v_scale, int v_scale_mode, const int32_t* block_table,
                   const int32_t* context_lens, int B, int next_n, int Hq, int Hkv, int D, int bs,
                   int64_t num_blocks, int max_blocks, float softmax_scale, int causal,
                   double* cond, double* vrange) {
  int group = Hq / Hkv;
  int max_len = max_blocks * bs;
  double fold_kmax = k_scale_mode == ORC_SCALE_PER_CHANNEL
                         ? (double)max_abs(k_scale, (int64_t)Hkv * D) : 0.0;
  int rc = 0;
  for (int b = 0; b < B; ++b)
    if (context_lens[b] > max_len) return -2;
#pragma omp parallel for schedule(dynamic)
  for (int u = 0; u < B * Hkv; ++u) {
    int b = u / Hkv, hk = u % Hkv;
    int L = context_lens[b];
    int n = L > 0 ? L : 1;
    float* kd = (float*)malloc(sizeof(float) * (size_t)n * D);
    float* vd = (float*)malloc(sizeof(float) * (size_t)n * D);
    double* csum = (double*)malloc(sizeof(double) * (size_t)n);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double* ab = (double*)malloc(sizeof(double) * (size_t)n);
    unsigned char* vis = (unsigned char*)malloc((size_t)n);
    float* qf = (float*)malloc(sizeof(float) * (size_t)D);
    int bad = gather_rows(kd, vd, csum, NULL, k_cache, v_cache, kv_kind, k_scale, k_scale_mode,
                          v_scale, v_scale_mode, block_table + (int64_t)b * max_blocks, L, hk, bs,
                          Hkv, D, num_blocks);
    if (bad) {
#pragma omp atomic write
      rc = -1;
    }
    for (int i = 0; i < next_n && !bad; ++i) {
      int pos = L - next_n + i;
      int nvis = L;
      if (causal && pos + 1 < nvis) nvis = pos + 1;
      for (int t = 0; t < L; ++t) vis[t] = t < nvis;
      for (int h = hk * group; h < (hk + 1) * group; ++h) {
        int64_t row = ((int64_t)b * next_n + i) * Hq + h;
        for (int d = 0; d < D; ++d) qf[d] = q_value(q, q_is_bf16, row * D + d);
        attend_row(out + row * D, qf, kd, vd, csum, vis, L, D, softmax_scale, s, ab,
                   cond ? cond + row * 4 : NULL, vrange ? vrange + row * 3 * D : NULL,
                   vrange ? vrange + row * 3 * D + D : NULL,
                   vrange ? vrange + row * 3 * D + 2 * D : NULL, fold_kmax);
      }
    }
    free(kd);
    free(vd);
    free(csum);
    free(s);
    free(ab);
    free(vis);
    free(qf);
  }
  return rc;
}

/* ------------------------------------------------------------------ */
/* Selection-driven sparse paged attention [P3] [P1]                   */
/* ------------------------------------------------------------------ */

/* mark[t] = 1 for every entry t of the topk entries of sel_row with
 * 0 <= t < L, else 0 (entries outside [0, L), -1 padding included, select
 * nothing; a repeated entry selects its token once). */
static void mark_selection(unsigned char* mark, const int32_t* sel_row, int topk, int L) {
  memset(mark, 0, (size_t)(L > 0 ? L : 1));
  for (int j = 0; j < topk; ++j)
    if (sel_row[j] >= 0 && sel_row[j] < L) mark[sel_row[j]] = 1;
}

/*
 * out[b, i, h, :] = softmax over the selected tokens S_{b,i} of
 * softmax_scale * q[b,i,h,:] . K_t, times V_t, summed over S_{b,i} in
 * ascending token order; dequantize first as in orc_paged_attn. S_{b,i} is the
 * set of sel[b, i, :] entries in [0, L_b) [P3, Investigation: the selected
 * token ids of a query row]. All heads of a row share its selection. An empty
 * selection gives +0. No causal limit is applied: the selection alone decides
 * what a row sees. Tokens outside every selection are never read, so tail
 * slots and the null block cannot reach the output [P1, Fix]. cond / vrange
 * as for orc_paged_attn, over each row's selected tokens.
 */
int orc_paged_attn_sparse(double* out, const uint16_t* q, int q_is_bf16, const uint8_t* k_cache,
                          const uint8_t* v_cache, int kv_kind, const float* k_scale,
                          int k_scale_mode, const float* v_scale, int v_scale_mode,
                          const int32_t* block_table, const int32_t* context_lens,
                          const int32_t* sel, int topk, int B, int next_n, int Hq, int Hkv, int D,
                          int bs, int64_t num_blocks, int max_blocks, float softmax_scale,
                          double* cond, double* vrange) {
  int group = Hq / Hkv;
  int max_len = max_blocks * bs;
  double fold_kmax = k_scale_mode == ORC_SCALE_PER_CHANNEL
                         ? (double)max_abs(k_scale, (int64_t)Hkv * D) : 0.0;
  int rc = 0;
  for (int b = 0; b < B; ++b)
    if (context_lens[b] > max_len) return -2;
#pragma omp parallel for schedule(dynamic)
  for (int u = 0; u < B * Hkv; ++u) {
    int b = u / Hkv, hk = u % Hkv;
    int L = context_lens[b];
    int n = L > 0 ? L : 1;
    float* kd = (float*)malloc(sizeof(float) * (size_t)n * D);
    float* vd = (float*)malloc(sizeof(float) * (size_t)n * D);
    double* csum = (double*)malloc(sizeof(double) * (size_t)n);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double* ab = (double*)malloc(sizeof(double) * (size_t)n);
    unsigned char* mark = (unsigned char*)malloc((size_t)n * (next_n > 0 ? next_n : 1));
    unsigned char* any = (unsigned char*)calloc((size_t)n, 1);
    float* qf = (float*)malloc(sizeof(float) * (size_t)D);
    for (int i = 0; i < next_n; ++i) {
      mark_selection(mark + (size_t)i * n, sel + ((int64_t)b * next_n + i) * topk, topk, L);
      for (int t = 0; t < L; ++t) any[t] |= mark[(size_t)i * n + t];
    }
    int bad = gather_rows(kd, vd, csum, any, k_cache, v_cache, kv_kind, k_scale, k_scale_mode,
                          v_scale, v_scale_mode, block_table + (int64_t)b * max_blocks, L, hk, bs,
                          Hkv, D, num_blocks);
    if (bad) {
#pragma omp atomic write
      rc = -1;
    }
    for (int i = 0; i < next_n && !bad; ++i) {
      for (int h = hk * group; h < (hk + 1) * group; ++h) {
        int64_t row = ((int64_t)b * next_n + i) * Hq + h;
        for (int d = 0; d < D; ++d) qf[d] = q_value(q, q_is_bf16, row * D + d);
        attend_row(out + row * D, qf, kd, vd, csum, mark + (size_t)i * n, L, D, softmax_scale,
                   s, ab, cond ? cond + row * 4 : NULL, vrange ? vrange + row * 3 * D : NULL,
                   vrange ? vrange + row * 3 * D + D : NULL,
                   vrange ? vrange + row * 3 * D + 2 * D : NULL, fold_kmax);
      }
    }
    free(kd);
    free(vd);
    free(csum);
    free(s);
    free(ab);
    free(mark);
    free(any);
    free(qf);
  }
  return rc;
}

/*
 * Grouped union plan of a selection [P3, Summary: the grouped planner keeps
 * its physical-page union and token masks, sorted with the logical page as the
 * key and the physical address as payload]: for sequence b, the logical pages
 * holding at least one selected token of any row, in ascending logical order;
 * entry e is {physical block, logical block} and mask[b, e, i] has bit j set
 * when row i selected token (logical block) * bs + j. count[b] is the number
 * of entries; entries are written up to cap per sequence (returns -3 when a
 * sequence needs more). Reading: one group per sequence (all its rows), so
 * the row-category and first-query keys of the pages' sort are constant and
 * the order is the logical page order.
 */
int orc_sparse_plan(int32_t* entries, uint32_t* masks, int32_t* count, const int32_t* sel,
                    int topk, const int32_t* block_table, const int32_t* context_lens, int B,
                    int next_n, int bs, int max_blocks, int cap) {
  if (next_n > 64 || bs > 32) return -1;
  int rc = 0;
  unsigned char* mark = (unsigned char*)malloc((size_t)(max_blocks * bs > 0 ? max_blocks * bs : 1) * 64);
  for (int b = 0; b < B; ++b) {
    int L = context_lens[b];
    if (L > max_blocks * bs) { rc = -2; break; }
    for (int i = 0; i < next_n; ++i)
      mark_selection(mark + (size_t)i * max_blocks * bs, sel + ((int64_t)b * next_n + i) * topk,
                     topk, L);
    int n = 0;
    for (int lp = 0; lp < max_blocks && lp * bs < L; ++lp) {
      uint32_t rowmask[64] = {0};
      int any = 0;
      for (int i = 0; i < next_n; ++i)
        for (int j = 0; j < bs && lp * bs + j < L; ++j)
          if (mark[(size_t)i * max_blocks * bs + lp * bs + j]) {
            rowmask[i] |= 1u << j;
            any = 1;
          }
      if (!any) continue;
      if (n >= cap) { rc = -3; break; }
      int64_t e = (int64_t)b * cap + n;
      entries[2 * e + 0] = block_table[(int64_t)b * max_blocks + lp];
      entries[2 * e + 1] = lp;
      for (int i = 0; i < next_n; ++i) masks[e * next_n + i] = rowmask[i];
      ++n;
    }
    if (rc) break;
    count[b] = n;
  }
  free(mark);
  return rc;
}

/* ------------------------------------------------------------------ */
/* MXFP4 paged MQA logits [P5]                                         */
/* ------------------------------------------------------------------ */

/*
 * Scale-factor slot that holds token t's scale bytes within a kv_fused block
 * [P5, is_kv_sf_interleaved]. In token order the slot is t. In the interleaved
 * order the block's slots are split into spi equal runs dealt round-robin, and
 * slot k holds token (k % spi) * (bs / spi) + k / spi (spi = scale bytes per
 * token, one int32 per slot); the slot of t is found by walking k through
 * that formula.
 */
static int sf_slot_of_token(int t, int bs, int spi, int interleaved) {
  if (!interleaved) return t;
  for (int k = 0; k < bs; ++k)
    if ((k % spi) * (bs / spi) + k / spi == t) return k;
  return -1;
}

/* Value x rounded to the epilogue type: fp32 (0), fp16 (1) or bf16 (2), both
 * round to nearest even. */
static float epi_round(float x, int epi_format) {
  if (epi_format == 1) return orc_f16_to_f32(orc_f64_to_f16((double)x));
  if (epi_format == 2) return orc_bf16_to_f32(orc_f32_to_bf16(x));
  return x;
}

/* One step of the weighted head chain [P5, epi_dtype]. fp32: fmaf(w, s, acc).
 * Reading for the fp16 / bf16 epilogues (the page names them without their
 * arithmetic): the weight and the head's dot product are rounded to the
 * epilogue type, the step is the fp32 fmaf of those and the running value, and
 * its result is rounded to the epilogue type again. */
static float epi_step(float w, float s, float acc, int epi_format) {
  return epi_round(fmaf(epi_round(w, epi_format), epi_round(s, epi_format), acc), epi_format);
}

/*
 * out[b*next_n + i, t] = sum over heads h (ascending, fp32 fmaf chain from +0)
 *   of weights[b*next_n + i, h] * A(S_h) (each step as epi_step), with
 *   S_h = sum over d (ascending, fp32) of deq(q[b,i,h,d]) * deq(k_t[d]),
 * for t < context_lens[b]; -inf for context_lens[b] <= t < max_context_len.
 * A is the identity, or with relu != 0 the rectifier (S_h > 0 ? S_h : +0).
 *
 * Layouts from the API page: q [B, next_n, H, D/2] two E2M1 per byte; sf_q
 * [B, next_n, H] int32 holding D/sf_vec UE8M0 bytes; kv_fused
 * [num_blocks, bs, 1, D/2 + D/sf_vec] where each block stores all tokens' FP4
 * data first and then all tokens' scale bytes, in token order, or with
 * sf_interleaved != 0 in the interleaved slot order (sf_slot_of_token);
 * weights [B*next_n, H] fp32. Readings: element 2j is the low nibble; byte g
 * of the int32 (bits 8g..8g+7) scales elements [g*sf_vec, (g+1)*sf_vec); the
 * pages name no activation, so A is the identity unless the caller asks for
 * the rectifier. The output is fp32 here; fp16 / bf16 outputs are the
 * round-to-nearest-even conversions of these values.
 */
int orc_mqa_logits(float* out, int64_t out_row_stride, const uint8_t* q, const int32_t* sf_q,
                   const uint8_t* kv_fused, const float* weights, const int32_t* context_lens,
                   const int32_t* block_table, int B, int next_n, int H, int D, int bs,
                   int max_blocks, int max_context_len, int sf_vec, int sf_interleaved,
                   int relu, int epi_format) {
  int row_bytes = D / 2 + D / sf_vec;
  int spi = D / sf_vec;
  if (sf_interleaved && bs % spi != 0) return -3;
  for (int b = 0; b < B; ++b)
    if (context_lens[b] > max_context_len || context_lens[b] > max_blocks * bs) return -2;
  /* rows are independent: one per OpenMP work unit */
#pragma omp parallel for schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    int L = context_lens[b];
    for (int i = 0; i < next_n; ++i) {
      int64_t r = (int64_t)b * next_n + i;
      float* orow = out + r * out_row_stride;
      for (int t = 0; t < L; ++t) {
        int64_t blk = block_table[(int64_t)b * max_blocks + t / bs];
        int slot = t % bs;
        const uint8_t* base = kv_fused + blk * (int64_t)bs * row_bytes;
        const uint8_t* kdata = base + (int64_t)slot * (D / 2);
        const uint8_t* ksf = base + (int64_t)bs * (D / 2) +
                             (int64_t)sf_slot_of_token(slot, bs, spi, sf_interleaved) * (D / sf_vec);
        float acc = 0.0f;
        for (int h = 0; h < H; ++h) {
          const uint8_t* qd = q + (r * H + h) * (D / 2);
          uint32_t qsf = (uint32_t)sf_q[r * H + h];
          float sh = 0.0f;
          for (int d = 0; d < D; ++d) {
            int g = d / sf_vec;
            uint8_t qb = qd[d / 2], kb = kdata[d / 2];
            float qv = orc_e2m1_to_f32((d % 2 == 0) ? (qb & 15) : (qb >> 4)) *
                       orc_ue8m0_to_f32((uint8_t)((qsf >> (8 * g)) & 0xFF));
            float kv = orc_e2m1_to_f32((d % 2 == 0) ? (kb & 15) : (kb >> 4)) *
                       orc_ue8m0_to_f32(ksf[g]);
            sh += qv * kv;
          }
          if (relu) sh = sh > 0.0f ? sh : 0.0f;
          acc = epi_step(weights[r * H + h], sh, acc, epi_format);
        }
        orow[t] = acc;
      }
      for (int t = L; t < max_context_len; ++t) orow[t] = -INFINITY;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Top-k token selection over logits [P3] [P5]                          */
/* ------------------------------------------------------------------ */

/* One logit of a row: fp32, fp16 (1) or bf16 (2) bits. */
static float logit_value(const void* logits, int fmt, int64_t idx) {
  if (fmt == 1) return orc_f16_to_f32(((const uint16_t*)logits)[idx]);
  if (fmt == 2) return orc_bf16_to_f32(((const uint16_t*)logits)[idx]);
  return ((const float*)logits)[idx];
}

typedef struct {
  float v;
  int32_t t;
} orc_scored;

/* Rank order of the selection: larger value first (equal values, -0 and +0
 * included, tie), NaN after every number, then the lower token id. */
static int rank_cmp(const void* pa, const void* pb) {
  const orc_scored* a = (const orc_scored*)pa;
  const orc_scored* b = (const orc_scored*)pb;
  int an = isnan(a->v), bn = isnan(b->v);
  if (an != bn) return an ? 1 : -1;
  if (!an && a->v != b->v) return a->v > b->v ? -1 : 1;
  return (a->t > b->t) - (a->t < b->t);
}

static int int_cmp(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/*
 * sel[r, :] for row r = b * next_n + i: the ids of the k highest logits of
 * row r among tokens t < context_lens[b] (the tokens the logits cover; the
 * -inf tail past the length is not a candidate), in ascending id order, then
 * -1 for the positions left when fewer than k tokens exist. This is the
 * top-k over the indexer logits that gives each query row its token set
 * [P3, Investigation: the selected token ids; Upstream check: top-k]. The
 * pages give no tie rule; the reading taken: equal logits go to the lower
 * token id, and NaN ranks below every number. Sorting is a library step
 * (qsort) under that total order.
 */
int orc_topk_select(int32_t* sel, const void* logits, int fmt, int64_t row_stride,
                    const int32_t* context_lens, int B, int next_n, int k) {
  int rc = 0;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < B * next_n; ++r) {
    int L = context_lens[r / next_n];
    if (L < 0 || (int64_t)L > row_stride) {
#pragma omp atomic write
      rc = -2;
      continue;
    }
    orc_scored* c = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)(L > 0 ? L : 1));
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    for (int t = 0; t < L; ++t) {
      c[t].v = logit_value(logits, fmt, (int64_t)r * row_stride + t);
      c[t].t = t;
    }
    qsort(c, (size_t)L, sizeof(orc_scored), rank_cmp);
    int n = L < k ? L : k;
    for (int j = 0; j < n; ++j) ids[j] = c[j].t;
    qsort(ids, (size_t)n, sizeof(int32_t), int_cmp);
    for (int j = 0; j < k; ++j) sel[(int64_t)r * k + j] = j < n ? ids[j] : -1;
    free(c);
    free(ids);
  }
  return rc;
}

/* fp32 -> bf16 bits of n values, round to nearest even (orc_f32_to_bf16). */
void orc_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------ */
/* KV insert [P4]                                                      */
/* ------------------------------------------------------------------ */

static float in_value(const uint16_t* x, int in_is_bf16, int64_t idx) {
  return in_is_bf16 ? orc_bf16_to_f32(x[idx]) : orc_f16_to_f32(x[idx]);
}

static void store_code(uint8_t* cache, int kind, int64_t blk, int off, int hk, int d, int bs,
                       int Hkv, int D, float x, float scale, uint16_t raw_bits) {
  int64_t row = (blk * bs + off) * Hkv + hk;
  int64_t row_bytes = (int64_t)D * elem_bits(kind) / 8;
  uint8_t* p = cache + row * row_bytes;
  if (kind == ORC_KV_F16 || kind == ORC_KV_BF16) {
    memcpy(p + 2 * d, &raw_bits, 2);
    return;
  }
  float y = x / scale; /* IEEE fp32 division */
  if (kind == ORC_KV_E4M3) {
    p[d] = orc_f32_to_e4m3(y);
  } else if (kind == ORC_KV_INT8) {
    p[d] = (uint8_t)(int8_t)orc_round_clamp(y, 127);
  } else {
    int nib = orc_round_clamp(y, 7) & 15;
    if (d % 2 == 0)
      p[d / 2] = (uint8_t)((p[d / 2] & 0xF0) | nib);
    else
      p[d / 2] = (uint8_t)((p[d / 2] & 0x0F) | (nib << 4));
  }
}

/*
 * Write rows k[i], v[i] ([T, Hkv, D]) of new tokens into the paged caches at
 * slot_mapping[i] (block = slot / bs, offset = slot % bs). Rows with
 * i >= num_slots or slot < 0 have no slot and are skipped, as the KV-only
 * insert skips padding rows that have no slot [P4, Design]; so are rows whose
 * slot lies past num_blocks * bs (reading: the pages say nothing of them, and
 * a write there would leave the cache). Codes: E4M3
 * nearest-even saturating, INT8/INT4 nearest-even clamped to +-127 / +-7,
 * computed from x / scale in fp32. F16/BF16 caches store the input bits
 * unchanged and require the matching input dtype.
 */
int orc_kv_insert(uint8_t* k_cache, uint8_t* v_cache, int kv_kind, const uint16_t* k,
                  const uint16_t* v, int in_is_bf16, const int64_t* slot_mapping, int64_t T,
                  int64_t num_slots, int Hkv, int D, int bs, int64_t num_blocks,
                  const float* k_scale, int k_scale_mode, const float* v_scale, int v_scale_mode) {
  for (int64_t i = 0; i < T; ++i) {
    if (i >= num_slots) continue;
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t blk = slot / bs;
    int off = (int)(slot % bs);
    if (blk >= num_blocks) continue; /* a slot past the cache is not written */
    for (int hk = 0; hk < Hkv; ++hk) {
      for (int d = 0; d < D; ++d) {
        int64_t idx = (i * Hkv + hk) * D + d;
        store_code(k_cache, kv_kind, blk, off, hk, d, bs, Hkv, D, in_value(k, in_is_bf16, idx),
                   scale_of(k_scale, k_scale_mode, hk, d, D), k[idx]);
        store_code(v_cache, kv_kind, blk, off, hk, d, bs, Hkv, D, in_value(v, in_is_bf16, idx),
                   scale_of(v_scale, v_scale_mode, hk, d, D), v[idx]);
      }
    }
  }
  return 0;
}

/*
 * MXFP4 insert into the kv_fused layout [P5, kv_fused; is_kv_sf_interleaved]:
 * row i of k ([T, D], fp16 or bf16) goes to token slot_mapping[i] (block =
 * slot / bs, position = slot % bs); rows with i >= num_slots or slot < 0 are
 * skipped [P4, Design]. Each group of sf_vec values takes the scale byte of
 * orc_mx_scale_byte and E2M1 codes of x / 2^(byte - 127) (an exact power-of-two
 * division); element 2j is the low nibble. The group bytes go to
 * [bs * D/2 data][bs * D/sf_vec scales] of the block, the scales of the token
 * at its token-order slot or its interleaved slot (sf_slot_of_token).
 */
int orc_mxfp4_insert(uint8_t* kv_fused, const uint16_t* k, int in_is_bf16,
                     const int64_t* slot_mapping, int64_t num_tokens, int64_t num_slots, int D,
                     int bs, int64_t num_blocks, int sf_vec, int sf_interleaved) {
  int spi = D / sf_vec;
  int64_t block_bytes = (int64_t)bs * (D / 2 + D / sf_vec);
  if (D % sf_vec != 0 || sf_vec % 2 != 0) return -1;
  if (sf_interleaved && bs % spi != 0) return -3;
  for (int64_t i = 0; i < num_tokens; ++i) {
    if (i >= num_slots) continue;
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t blk = slot / bs;
    int pos = (int)(slot % bs);
    if (blk >= num_blocks) return -2;
    uint8_t* base = kv_fused + blk * block_bytes;
    uint8_t* data = base + (int64_t)pos * (D / 2);
    uint8_t* sf = base + (int64_t)bs * (D / 2) +
                  (int64_t)sf_slot_of_token(pos, bs, spi, sf_interleaved) * spi;
    for (int g = 0; g < spi; ++g) {
      float amax = 0.0f;
      for (int j = 0; j < sf_vec; ++j) {
        float x = in_value(k, in_is_bf16, i * D + g * sf_vec + j);
        if (fabsf(x) > amax) amax = fabsf(x);
      }
      uint8_t byte = orc_mx_scale_byte(amax);
      sf[g] = byte;
      for (int j = 0; j < sf_vec; ++j) {
        int d = g * sf_vec + j;
        float x = in_value(k, in_is_bf16, i * D + d);
        uint8_t c = orc_f32_to_e2m1(ldexpf(x, 127 - (int)byte));
        if (d % 2 == 0)
          data[d / 2] = (uint8_t)((data[d / 2] & 0xF0) | c);
        else
          data[d / 2] = (uint8_t)((data[d / 2] & 0x0F) | (c << 4));
      }
    }
  }
  return 0;
}
