// pa_attn_bf16.hip -- paged attention ring kernels for BF16 KV caches.
#include "pa_attn.hpp"

namespace pa {

RingFn pick_ring_bf16(int D, int nw, int RT, int qf, int mode) {
  return pick_d<PA_KV_BF16>(D, nw, RT, qf, mode);
}

PrefillFn pick_prefill_bf16(int D, bool fold) { return pick_prefill<PA_KV_BF16>(D, fold); }

}  // namespace pa
