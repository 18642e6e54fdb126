// pa_attn_int4.hip -- paged attention ring kernels for INT4 KV caches.
#include "pa_attn.hpp"

namespace pa {

RingFn pick_ring_int4(int D, int nw, int RT, int qf, int mode) {
  return pick_d<PA_KV_INT4>(D, nw, RT, qf, mode);
}

PrefillFn pick_prefill_int4(int D, bool fold) { return pick_prefill<PA_KV_INT4>(D, fold); }

}  // namespace pa
