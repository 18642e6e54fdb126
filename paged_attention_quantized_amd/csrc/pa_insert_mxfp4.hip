// pa_insert_mxfp4.hip -- MXFP4 insert into the kv_fused cache of the paged MQA
// logits ["flashinfer.fp4_paged_mqa_logits" API page: kv_fused,
// is_kv_sf_interleaved], on gfx950.
//
// A wavefront takes 2 token rows of 128 values (their slots and inputs are all
// loaded first); lane l holds elements 2l and 2l + 1 of a row, so a 32-value
// scale group is exactly one 16-lane row of the wave. Per group:
// the largest magnitude (a max over the row), the UE8M0 byte max(0, E - 2)
// where E is the fp32 exponent field of that magnitude (the shared scale
// 2^(floor(log2 amax) - 2) of the OCP Microscaling rule; an all-zero group gets
// byte 0), then each value times 2^(127 - byte) (exact) rounded to the E2M1
// grid with ties to the even code and saturation at 6. The lane's two codes
// form one byte (element 2l in the low nibble); the 64 bytes of the row and
// the 4 scale bytes go to the token's block position and scale slot.
#include "pa_device.hpp"
#include "pa_host.hpp"

namespace pa {

struct Mxfp4InsertParams {
  uint8_t* kv;
  const uint32_t* k;  // two 16-bit values per dword
  const int64_t* slot_mapping;
  int64_t num_tokens, num_slots, num_blocks;
  int bs, sfi;
};

// E2M1 magnitude code of a >= 0: the number of grid midpoints below it, a
// midpoint itself going to the neighbour whose code is even.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

template <bool BF16>
__device__ __forceinline__ float in_f32(uint32_t half_bits) {
  if constexpr (BF16)
    return __uint_as_float(half_bits << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)half_bits);
}

#ifndef MX_ROWS_PER_WAVE
#define MX_ROWS_PER_WAVE 2
#endif
constexpr int kRowsPerWave = MX_ROWS_PER_WAVE;

template <bool BF16>
__global__ __launch_bounds__(256) void mxfp4_insert_kernel(Mxfp4InsertParams p) {
  constexpr int D = 128, ROWB = D / 2, SFB = D / 32, R = kRowsPerWave;
  const int lane = threadIdx.x & 63;
  const int64_t i0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  const int64_t rows = p.num_tokens < p.num_slots ? p.num_tokens : p.num_slots;
  // every load of the wave's rows first: slots, then the input dwords
  int64_t slot[R];
  uint32_t w[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = i0 + r;
    slot[r] = i < rows ? p.slot_mapping[i] : -1;  // rows past the slot list have no slot [INSERT]
    w[r] = i < rows ? p.k[i * (D / 2) + lane] : 0u;
  }
  const int q = p.bs / SFB;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t blk = slot[r] / p.bs;
    // padding rows carry slot -1; a slot outside the cache is never written
    if (slot[r] < 0 || blk >= p.num_blocks) continue;
    const int pos = (int)(slot[r] % p.bs);
    const float x0 = in_f32<BF16>(w[r] & 0xFFFFu), x1 = in_f32<BF16>(w[r] >> 16);
    // largest magnitude of the lane's 16-lane row (its 32-value group): DPP
    // rotations by 1, 2, 4, 8 inside the row leave the row max in every lane
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x121, 0xf, 0xf, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x122, 0xf, 0xf, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x124, 0xf, 0xf, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x128, 0xf, 0xf, false)));
    const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    const int sbyte = ebits >= 2 ? ebits - 2 : 0;
    const int sh = 127 - sbyte;
    const float y0 = __builtin_amdgcn_ldexpf(x0, sh), y1 = __builtin_amdgcn_ldexpf(x1, sh);
    const uint32_t c0 = e2m1_mag(fabsf(y0)) | (__builtin_signbit(y0) ? 8u : 0u);
    const uint32_t c1 = e2m1_mag(fabsf(y1)) | (__builtin_signbit(y1) ? 8u : 0u);
    uint8_t* base = p.kv + (size_t)blk * p.bs * (ROWB + SFB);
    base[(size_t)pos * ROWB + lane] = (uint8_t)(c0 | (c1 << 4));
    // scale slot: token order, or slot k holding token (k % 4) * (bs / 4) + k / 4
    const int sslot = p.sfi ? SFB * (pos % q) + pos / q : pos;
    if ((lane & 15) == 0) base[(size_t)p.bs * ROWB + sslot * SFB + (lane >> 4)] = (uint8_t)sbyte;
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status kv_insert_mxfp4(const pa_mxfp4_insert_args* a, void* stream) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "kv_insert_mxfp4: args is NULL");
  if (a->num_tokens < 0 || a->num_slots < 0 || a->num_blocks < 1 || a->block_size < 1)
    return fail(PA_ERR_INVALID_ARG, "kv_insert_mxfp4: bad sizes");
  if (a->head_dim != 128 || a->sf_vec_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "kv_insert_mxfp4: head_dim must be 128, sf_vec_size 32");
  if (a->block_size % 4 != 0)
    return fail(PA_ERR_UNSUPPORTED, "kv_insert_mxfp4: block_size must be a multiple of 4");
  if (a->in_dtype != PA_DT_F16 && a->in_dtype != PA_DT_BF16)
    return fail(PA_ERR_UNSUPPORTED, "kv_insert_mxfp4: input must be fp16 or bf16");
  if (a->sf_interleaved != 0 && a->sf_interleaved != 1)
    return fail(PA_ERR_INVALID_ARG, "kv_insert_mxfp4: sf_interleaved must be 0 or 1");
  const int64_t rows = a->num_tokens < a->num_slots ? a->num_tokens : a->num_slots;
  if (rows == 0) return PA_OK;
  if (!a->kv_fused || !a->k || !a->slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "kv_insert_mxfp4: null pointer");
  Mxfp4InsertParams p;
  p.kv = a->kv_fused;
  p.k = (const uint32_t*)a->k;
  p.slot_mapping = a->slot_mapping;
  p.num_tokens = a->num_tokens;
  p.num_slots = a->num_slots;
  p.num_blocks = a->num_blocks;
  p.bs = a->block_size;
  p.sfi = a->sf_interleaved;
  const dim3 grid((unsigned)ceil_div(rows, 4 * kRowsPerWave));
  hipStream_t s = (hipStream_t)stream;
  if (a->in_dtype == PA_DT_BF16)
    launch_timed(mxfp4_insert_kernel<true>, grid, dim3(256), s, p);
  else
    launch_timed(mxfp4_insert_kernel<false>, grid, dim3(256), s, p);
  return launch_status("kv_insert_mxfp4 kernel");
}
