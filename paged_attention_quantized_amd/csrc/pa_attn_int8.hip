// pa_attn_int8.hip -- paged attention ring kernels for INT8 KV caches.
#include "pa_attn.hpp"

namespace pa {

RingFn pick_ring_int8(int D, int nw, int RT, int qf, int mode) {
  return pick_d<PA_KV_INT8>(D, nw, RT, qf, mode);
}

PrefillFn pick_prefill_int8(int D, bool fold) { return pick_prefill<PA_KV_INT8>(D, fold); }

}  // namespace pa
