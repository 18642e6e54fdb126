// pa_logits.hip -- MXFP4 paged MQA logits (placeholder until the kernel lands).
#include "pa_host.hpp"

using namespace pa;

extern "C" size_t paged_mqa_logits_workspace_size(const pa_logits_args* a) {
  (void)a;
  return 0;
}

extern "C" pa_status paged_mqa_logits(const pa_logits_args* a, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  (void)a; (void)workspace; (void)workspace_bytes; (void)stream;
  return fail(PA_ERR_UNSUPPORTED, "paged_mqa_logits: not built yet");
}
