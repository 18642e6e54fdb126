// pa_device.hpp -- device helpers shared by the gfx950 kernels of libpa:
// vector types, KV-cache codecs (code -> fp16) and small wavefront utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ __forceinline__ uint32_t as_u32(h2 x) { return __builtin_bit_cast(uint32_t, x); }

// ---------------------------------------------------------------------------
// Cache element kinds. Every decode is exact: E4M3, INT8 and INT4 codes are all
// representable in fp16 ([NULLPAD] E4M3 NaN bytes 0x7F/0xFF decode to fp16 NaN).
// ---------------------------------------------------------------------------

template <int KIND>
struct Kv;

// fp16 cache: 2 bytes per element, no decode.
template <>
struct Kv<PA_KV_F16> {
  static constexpr int kBits = 16;
  // one dword -> one pair, natural order
  static constexpr int kPairsPerDword = 1;
  __device__ static void decode(uint32_t w, h2* out) { out[0] = as_h2(w); }
  // element order of the pairs produced from one dword (see decode)
  __device__ static constexpr int order(int e) { return e; }
};

// bf16 cache: 2 bytes per element; each value is widened to fp32 (its upper
// half) and converted to fp16 toward zero. bf16's 8-bit significand fits
// fp16's 11 bits, so the conversion is exact for magnitudes in fp16's normal
// range [2^-14, 65504]; smaller ones keep fp16's subnormal precision, larger
// finite ones become +-65504, and infinities and NaN stay what they are.
template <>
struct Kv<PA_KV_BF16> {
  static constexpr int kBits = 16;
  static constexpr int kPairsPerDword = 1;
  __device__ static void decode(uint32_t w, h2* out) {
    out[0] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                __uint_as_float(w & 0xFFFF0000u)));
  }
  __device__ static constexpr int order(int e) { return e; }
};

// OCP FP8 E4M3FN via the gfx950 scaled fp8 -> fp16 conversion (scale 1.0):
// bytes (0,1) and (2,3) of a dword become two fp16 pairs.
template <>
struct Kv<PA_KV_E4M3> {
  static constexpr int kBits = 8;
  static constexpr int kPairsPerDword = 2;
  __device__ static void decode(uint32_t w, h2* out) {
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  }
  __device__ static constexpr int order(int e) { return e; }
};

// INT8: bias each byte to unsigned (x ^ 0x80), place it under the fp16
// exponent of 1024 (0x64xx = 1024 + byte) and subtract 1024 + 128.
template <>
struct Kv<PA_KV_INT8> {
  static constexpr int kBits = 8;
  static constexpr int kPairsPerDword = 2;
  __device__ static void decode(uint32_t w, h2* out) {
    uint32_t x = w ^ 0x80808080u;
    uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
    uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    out[0] = as_h2(lo) - bias;
    out[1] = as_h2(hi) - bias;
  }
  __device__ static constexpr int order(int e) { return e; }
};

// INT4: eight signed nibbles per dword (element k at bits 4k..4k+3). Flipping
// bit 3 of a nibble maps value v to u = v + 8 in [0, 15]. Nibbles k and k + 4
// (k = 0, 2) are masked into bits 0-3 of each fp16 half under the exponent of
// 1024, and 1032 is subtracted; nibbles k = 1, 3 are masked in place (bits
// 4-7: the half reads 1024 + 16 u) and one fma takes x / 16 - 72 = u - 8 (every
// step exact). Mask, flip and exponent are one 3-input bitwise op,
// (s & mask) ^ (exponent | flip) (the exponent bits are zero after the mask,
// so the xor sets them), and only the upper byte pair needs a shift: 9
// instructions per 8 values. The pairs come out as (e0,e4), (e1,e5), (e2,e6),
// (e3,e7).
template <>
struct Kv<PA_KV_INT4> {
  static constexpr int kBits = 4;
  static constexpr int kPairsPerDword = 4;
  __device__ static void decode(uint32_t w, h2* out) {
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    // truth table 0x6A: (a & b) ^ c, a = the codes, b = mask, c = exponent | flip
    out[0] = as_h2(__builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, 0x6A)) - bias;
    out[1] = __builtin_elementwise_fma(
        as_h2(__builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, 0x6A)), sixteenth, bias16);
    out[2] = as_h2(__builtin_amdgcn_bitop3_b32(w8, 0x000F000Fu, 0x64086408u, 0x6A)) - bias;
    out[3] = __builtin_elementwise_fma(
        as_h2(__builtin_amdgcn_bitop3_b32(w8, 0x00F000F0u, 0x64806480u, 0x6A)), sixteenth, bias16);
  }
  // slot e of the 8 fp16 values produced from one dword holds element order(e)
  __device__ static constexpr int order(int e) { return (e >> 1) + 4 * (e & 1); }
};

// Decode a run of dwords into fp16 values. Slot s of the output holds element
// (s / (2 * kPairsPerDword)) * (2 * kPairsPerDword) + Kv::order(s % (2*kPairsPerDword))
// of the run.
template <int KIND, int NDW>
__device__ __forceinline__ void decode_run(const uint32_t* w, _Float16* out) {
  constexpr int P = Kv<KIND>::kPairsPerDword;
#pragma unroll
  for (int i = 0; i < NDW; ++i) {
    h2 pr[P];
    Kv<KIND>::decode(w[i], pr);
#pragma unroll
    for (int k = 0; k < P; ++k) {
      out[(i * P + k) * 2 + 0] = pr[k][0];
      out[(i * P + k) * 2 + 1] = pr[k][1];
    }
  }
}

// element index (within the run) of output slot s of decode_run
template <int KIND>
__device__ __forceinline__ constexpr int run_elem(int s) {
  constexpr int E = 2 * Kv<KIND>::kPairsPerDword;
  return (s / E) * E + Kv<KIND>::order(s % E);
}

// ---------------------------------------------------------------------------
// wavefront helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): shifts by 1, 2, 4, 8 inside each row of 16 lanes (lanes whose
// source falls outside the row read 0), then lane 15 of rows 0 and 2 is added
// to rows 1 and 3, and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Value of lane `l` (wave-uniform) in every lane.
__device__ __forceinline__ int lane_val(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// wave-uniform values, said so to the compiler (kept in SGPRs)
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uni64(uint64_t x) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32);
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4,
// scalar-base form): lane i of the wave writes lds + 16 * i, reading
// sbase + voff; lds and sbase are wave-uniform. The load is issued through
// inline asm so that the compiler does not treat the asynchronous LDS write as
// something every later LDS read has to wait for (it would wait for the whole
// ring); the ring's own vmcnt + barrier protocol orders writes and reads. The
// asm sets M0 itself; nothing else in these kernels uses M0. An LDS DMA that
// reads M0 right after a scalar write of M0 needs one wait state on gfx950
// (the compiler puts an s_nop between the pair when it emits them itself), so
// the asm carries it too.
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, const uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  // the base is uniform by construction; saying so keeps it in SGPRs
  const uint64_t sb = uni64((uint64_t)(uintptr_t)sbase);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0v),
               "v"(voff), "s"(sb)
               : "memory");
}




}  // namespace pa
