// pa_attn_f16.hip -- paged attention ring kernels for fp16 KV caches.
#include "pa_attn.hpp"

namespace pa {

RingFn pick_ring_f16(int D, int nw, int RT, int qf, int mode) {
  return pick_d<PA_KV_F16>(D, nw, RT, qf, mode);
}

PrefillFn pick_prefill_f16(int D, bool fold) { return pick_prefill<PA_KV_F16>(D, fold); }

}  // namespace pa
