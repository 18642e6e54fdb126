"""paged_attn_fwd_noalloc (the entry point for callers that cannot allocate)
against paged_attn_fwd, through the C ABI: two calls in a row on the library's
scratch array, the second with a smaller input, each equal to the
workspace-taking entry point's output bit for bit (and so within the 2e-3 /
1-ulp bar of the oracle comparison those outputs pass); a call that needs more
workspace than the array holds is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import DevAttn, compare_attn, oracle_attn, say

pytestmark = pytest.mark.gpu


def cases():
    rng = np.random.default_rng(4401)
    big = W.attn_case("noalloc_big", 4401, B=6, next_n=4, Hq=32, Hkv=8, D=128, bs=16,
                      lens=list(rng.integers(100, 1500, 6)), kv_kind=W.KV_E4M3,
                      scale_mode=W.SCALE_PER_TENSOR)
    small = W.attn_case("noalloc_small", 4402, B=2, next_n=1, Hq=16, Hkv=2, D=256, bs=32,
                        lens=[300, 41], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                        q_dist=(-100.0, 100.0), zero_k_channel_frac=0.1,
                        v_scale_range=(1e-2, 65504.0 / 127))
    return big, small


def run_noalloc(pa, d):
    c = d.case
    out = torch.full(c.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    pa.paged_attn_fwd_noalloc(out, d.q, d.k, d.v, d.bt, d.cl, c.max_context_len,
                              kv_kind=c.kv_kind, k_scale=d.ks, v_scale=d.vs,
                              k_scale_mode=c.k_scale_mode, v_scale_mode=c.v_scale_mode,
                              softmax_scale=c.softmax_scale, causal=c.causal)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_workspace_entry_point(pa):
    for case in cases():  # the second call is the smaller input
        d = DevAttn(case)
        say(f"noalloc {case.name} B={case.batch}")
        got = run_noalloc(pa, d)
        ref = d.run(pa).cpu().numpy()
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), case.name
        compare_attn(got, oracle_attn(case), case.name)


def test_noalloc_refuses_oversized_call(pa):
    # a chunked-prefill shape: 2048 query rows per KV head over 8 sequences
    case = W.attn_case("noalloc_huge", 4403, B=8, next_n=256, Hq=64, Hkv=8, D=128, bs=32,
                       lens=[300] * 8, kv_kind=W.KV_F16, scale_mode=W.SCALE_NONE)
    d = DevAttn(case)
    lib = pa.load()
    need = pa.paged_attn_workspace_size(d.q, d.k, d.bt, case.max_context_len, case.kv_kind)
    assert need > lib.paged_attn_noalloc_scratch_bytes()
    out = torch.empty(case.q.shape, dtype=torch.float16, device="cuda")
    say("noalloc oversized call")
    with pytest.raises(pa.PaError, match="WORKSPACE"):
        pa.paged_attn_fwd_noalloc(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len,
                                  kv_kind=case.kv_kind)
