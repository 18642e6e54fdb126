// pa_attn_e4m3.hip -- paged attention ring kernels for OCP FP8 E4M3 KV caches.
#include "pa_attn.hpp"

namespace pa {

RingFn pick_ring_e4m3(int D, int nw, int RT, int qf, int mode) {
  return pick_d<PA_KV_E4M3>(D, nw, RT, qf, mode);
}

PrefillFn pick_prefill_e4m3(int D, bool fold) { return pick_prefill<PA_KV_E4M3>(D, fold); }

}  // namespace pa
