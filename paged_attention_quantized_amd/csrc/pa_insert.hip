// pa_insert.hip -- paged KV insert (quantize new rows into the cache at their
// slots) and the codec probe pa_dequantize, on gfx950.
#include <math.h>

#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

// Nearest E4M3 code with ties to even, saturating to +-448; NaN -> 0x7F.
// Below 2^-6 the code spacing is 2^-9 (subnormals); in binade [2^e, 2^(e+1))
// it is 2^(e-3). Scaling by powers of two is exact, rintf rounds half to even,
// and the code of a value is monotone in it, so a rounded-up mantissa of 16
// simply carries into the next binade.
__device__ __forceinline__ uint32_t enc_e4m3(float y) {
  if (y != y) return 0x7Fu;
  const uint32_t sign = __builtin_signbit(y) ? 0x80u : 0u;
  const float a = fabsf(y);
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0x1p-6f) return sign | (uint32_t)rintf(a * 512.f);
  const int e = ilogbf(a);
  const int nm = (int)rintf(ldexpf(a, 3 - e));  // in [8, 16]
  return sign | (uint32_t)(((e + 7) << 3) + nm - 8);
}

__device__ __forceinline__ int enc_int(float y, float lim) {
  if (y != y) return 0;
  return (int)fminf(fmaxf(rintf(y), -lim), lim);
}

struct InsertParams {
  uint8_t* k_cache;
  uint8_t* v_cache;
  const uint16_t* k;  // fp16 or bf16 bits (in_bf16)
  const uint16_t* v;
  const int64_t* slot_mapping;
  const float* k_scale;
  const float* v_scale;
  int64_t num_tokens, num_slots, num_blocks;
  int Hkv, D, bs, k_mode, v_mode, in_bf16;
};

// Input value: fp16 bits, or bf16 bits (the upper half of an fp32).
__device__ __forceinline__ float in_val(const uint16_t* x, int d, bool bf16) {
  return bf16 ? __uint_as_float((uint32_t)x[d] << 16) : (float)__builtin_bit_cast(_Float16, x[d]);
}

__device__ __forceinline__ float scale_at(const float* s, int mode, int hk, int d, int D) {
  return mode == PA_SCALE_PER_TENSOR ? s[0] : (mode == PA_SCALE_PER_CHANNEL ? s[hk * D + d] : 1.f);
}

// One workgroup of 64 threads per (token, kv head); each thread writes whole
// bytes of the destination row (two elements for INT4).
template <int KIND>
__global__ __launch_bounds__(64) void insert_kernel(InsertParams p) {
  const int64_t i = blockIdx.x / p.Hkv;
  const int hk = blockIdx.x % p.Hkv;
  if (i >= p.num_slots) return;  // rows past the slot list have no slot [INSERT]
  const int64_t slot = p.slot_mapping[i];
  if (slot < 0) return;          // padding rows carry slot -1
  const int64_t blk = slot / p.bs;
  if (blk >= p.num_blocks) return;  // a slot past the cache is not written
  const int off = (int)(slot % p.bs);
  constexpr int BITS = Kv<KIND>::kBits;
  const int rb = p.D * BITS / 8;
  const size_t row = ((size_t)blk * p.bs + off) * p.Hkv + hk;
  const size_t src = ((size_t)i * p.Hkv + hk) * p.D;
  for (int plane = 0; plane < 2; ++plane) {
    uint8_t* dst = (plane ? p.v_cache : p.k_cache) + row * rb;
    const uint16_t* x = (plane ? p.v : p.k) + src;
    const float* sc = plane ? p.v_scale : p.k_scale;
    const int mode = plane ? p.v_mode : p.k_mode;
    const bool bf = p.in_bf16;
    if constexpr (KIND == PA_KV_F16 || KIND == PA_KV_BF16) {
      // the input bits unchanged (the input type matches the cache's)
      uint16_t* ds = reinterpret_cast<uint16_t*>(dst);
      for (int d = threadIdx.x; d < p.D; d += 64) ds[d] = x[d];
    } else if constexpr (KIND == PA_KV_INT4) {
      for (int j = threadIdx.x; j < rb; j += 64) {
        const int d = 2 * j;
        const int lo = enc_int(in_val(x, d, bf) / scale_at(sc, mode, hk, d, p.D), 7.f);
        const int hi = enc_int(in_val(x, d + 1, bf) / scale_at(sc, mode, hk, d + 1, p.D), 7.f);
        dst[j] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
      }
    } else {
      for (int d = threadIdx.x; d < p.D; d += 64) {
        const float y = in_val(x, d, bf) / scale_at(sc, mode, hk, d, p.D);
        dst[d] = KIND == PA_KV_E4M3 ? (uint8_t)enc_e4m3(y) : (uint8_t)(int8_t)enc_int(y, 127.f);
      }
    }
  }
}

// Codec probe: each thread decodes one dword of codes with the same decoder
// the attention kernel uses, then multiplies by the scale in fp32.
template <int KIND>
__global__ void dequant_kernel(const uint32_t* codes, int64_t ndw, const float* scale, int mode,
                               int64_t channels, float* out) {
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= ndw) return;
  constexpr int E = 2 * Kv<KIND>::kPairsPerDword;
  _Float16 hv[E];
  const uint32_t dw = codes[w];
  decode_run<KIND, 1>(&dw, hv);
#pragma unroll
  for (int s = 0; s < E; ++s) {
    const int64_t idx = w * E + run_elem<KIND>(s);
    float sc = 1.f;
    if (mode == PA_SCALE_PER_TENSOR) sc = scale[0];
    if (mode == PA_SCALE_PER_CHANNEL) sc = scale[idx % channels];
    out[idx] = (float)hv[s] * sc;
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status kv_insert(const pa_insert_args* a, void* stream) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "kv_insert: args is NULL");
  if (!valid_kind(a->kv_kind) || !valid_mode(a->k_scale_mode) || !valid_mode(a->v_scale_mode))
    return fail(PA_ERR_INVALID_ARG, "kv_insert: unknown kv_kind or scale mode");
  if (a->num_tokens < 0 || a->num_slots < 0 || a->num_kv_heads < 1 || a->head_dim < 2 ||
      a->block_size < 1 || a->num_blocks < 1 || (a->head_dim & 1))
    return fail(PA_ERR_INVALID_ARG, "kv_insert: bad sizes");
  if (a->in_dtype != PA_DT_F16 && a->in_dtype != PA_DT_BF16)
    return fail(PA_ERR_UNSUPPORTED, "kv_insert: in_dtype must be F16 or BF16");
  if ((a->kv_kind == PA_KV_F16 && a->in_dtype != PA_DT_F16) ||
      (a->kv_kind == PA_KV_BF16 && a->in_dtype != PA_DT_BF16))
    return fail(PA_ERR_UNSUPPORTED, "kv_insert: an F16 / BF16 cache takes input of its own type");
  if ((a->kv_kind == PA_KV_F16 || a->kv_kind == PA_KV_BF16) &&
      (a->k_scale_mode != PA_SCALE_NONE || a->v_scale_mode != PA_SCALE_NONE))
    return fail(PA_ERR_UNSUPPORTED, "kv_insert: F16 / BF16 KV takes no scales");
  const int64_t rows = a->num_tokens < a->num_slots ? a->num_tokens : a->num_slots;
  if (rows == 0) return PA_OK;
  if (!a->k_cache || !a->v_cache || !a->k || !a->v || !a->slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "kv_insert: null pointer");
  if ((a->k_scale_mode != PA_SCALE_NONE && !a->k_scale) ||
      (a->v_scale_mode != PA_SCALE_NONE && !a->v_scale))
    return fail(PA_ERR_INVALID_ARG, "kv_insert: scale mode set but scale pointer is NULL");
  InsertParams p;
  p.k_cache = (uint8_t*)a->k_cache;
  p.v_cache = (uint8_t*)a->v_cache;
  p.k = (const uint16_t*)a->k;
  p.v = (const uint16_t*)a->v;
  p.in_bf16 = a->in_dtype == PA_DT_BF16;
  p.num_blocks = a->num_blocks;
  p.slot_mapping = a->slot_mapping;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.num_tokens = a->num_tokens;
  p.num_slots = a->num_slots;
  p.Hkv = a->num_kv_heads;
  p.D = a->head_dim;
  p.bs = a->block_size;
  p.k_mode = a->k_scale_mode;
  p.v_mode = a->v_scale_mode;
  const dim3 grid((unsigned)(rows * a->num_kv_heads));
  hipStream_t s = (hipStream_t)stream;
  switch (a->kv_kind) {
    case PA_KV_F16: hipLaunchKernelGGL(insert_kernel<PA_KV_F16>, grid, dim3(64), 0, s, p); break;
    case PA_KV_BF16: hipLaunchKernelGGL(insert_kernel<PA_KV_BF16>, grid, dim3(64), 0, s, p); break;
    case PA_KV_E4M3: hipLaunchKernelGGL(insert_kernel<PA_KV_E4M3>, grid, dim3(64), 0, s, p); break;
    case PA_KV_INT8: hipLaunchKernelGGL(insert_kernel<PA_KV_INT8>, grid, dim3(64), 0, s, p); break;
    case PA_KV_INT4: hipLaunchKernelGGL(insert_kernel<PA_KV_INT4>, grid, dim3(64), 0, s, p); break;
    default: return fail(PA_ERR_UNSUPPORTED, "kv_insert: kind");
  }
  return launch_status("kv_insert kernel");
}

extern "C" pa_status pa_dequantize(pa_kv_kind kind, const void* codes, int64_t n,
                                   const float* scale, pa_scale_mode mode, int64_t channels,
                                   float* out, void* stream) {
  if (!valid_kind(kind) || !valid_mode(mode)) return fail(PA_ERR_INVALID_ARG, "pa_dequantize: kind");
  if (n < 0 || (mode == PA_SCALE_PER_CHANNEL && channels < 1))
    return fail(PA_ERR_INVALID_ARG, "pa_dequantize: bad sizes");
  const int64_t bits = kv_bits(kind);
  if ((n * bits) % 32) return fail(PA_ERR_INVALID_ARG, "pa_dequantize: n codes must fill dwords");
  if (n == 0) return PA_OK;
  if (!codes || !out || (mode != PA_SCALE_NONE && !scale))
    return fail(PA_ERR_INVALID_ARG, "pa_dequantize: null pointer");
  const int64_t ndw = n * bits / 32;
  const dim3 grid((unsigned)ceil_div(ndw, 256));
  hipStream_t s = (hipStream_t)stream;
  const uint32_t* c = (const uint32_t*)codes;
  switch (kind) {
    case PA_KV_F16: hipLaunchKernelGGL(dequant_kernel<PA_KV_F16>, grid, dim3(256), 0, s, c, ndw, scale, (int)mode, channels, out); break;
    case PA_KV_BF16: hipLaunchKernelGGL(dequant_kernel<PA_KV_BF16>, grid, dim3(256), 0, s, c, ndw, scale, (int)mode, channels, out); break;
    case PA_KV_E4M3: hipLaunchKernelGGL(dequant_kernel<PA_KV_E4M3>, grid, dim3(256), 0, s, c, ndw, scale, (int)mode, channels, out); break;
    case PA_KV_INT8: hipLaunchKernelGGL(dequant_kernel<PA_KV_INT8>, grid, dim3(256), 0, s, c, ndw, scale, (int)mode, channels, out); break;
    case PA_KV_INT4: hipLaunchKernelGGL(dequant_kernel<PA_KV_INT4>, grid, dim3(256), 0, s, c, ndw, scale, (int)mode, channels, out); break;
    default: return fail(PA_ERR_UNSUPPORTED, "pa_dequantize: kind");
  }
  return launch_status("pa_dequantize kernel");
}
