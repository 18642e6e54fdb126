// pa_attn_int8.hip -- paged attention ring kernels for INT8 KV caches.
#include "pa_attn.hpp"

namespace pa {

RingFn pick_ring_int8(int D, int nw, int RT, int hilo, int mode) {
  return pick_d<PA_KV_INT8>(D, nw, RT, hilo, mode);
}

PrefillFn pick_prefill_int8(int D, bool hilo) { return pick_prefill<PA_KV_INT8>(D, hilo); }

}  // namespace pa
