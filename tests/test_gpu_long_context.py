"""Long contexts: sequences of 70K to 200K tokens (a few narrow heads so the
inputs stay small) through the dense ring, the multi-row verify layout and the
sparse route, against the oracle; the sparse case's union reaches 12 500 pages.
Long runs cross many workgroup ranges, so the merge combines many partials per
(sequence, head)."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import DevAttn, compare_attn, dev, run_attn, say

pytestmark = pytest.mark.gpu


def _oracle(case):
    return oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                             case.context_lens, **case.oracle_kwargs())


LONG = [
    ("decode_fp8", dict(B=2, next_n=1, Hq=8, Hkv=1, D=128, bs=16, lens=[131072, 70001],
                        kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)),
    ("verify_int8", dict(B=2, next_n=4, Hq=8, Hkv=1, D=128, bs=32, lens=[100003, 4],
                         kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_TENSOR)),
    ("decode_f16", dict(B=1, next_n=1, Hq=4, Hkv=1, D=64, bs=16, lens=[200000],
                        kv_kind=W.KV_F16, scale_mode=W.SCALE_NONE)),
]


@pytest.mark.parametrize("idx", range(len(LONG)))
def test_long_context_parity(pa, idx):
    name, kw = LONG[idx]
    case = W.attn_case("long_" + name, 8201 + idx, **kw)
    say(f"long context {name} L={list(case.context_lens)}")
    got = run_attn(pa, case)
    r = compare_attn(got, _oracle(case), case.name)
    say(f"long context {name}: max err/tol = {r:.3f}")


def test_long_context_sparse(pa):
    """200K tokens in pages of 16 (12 500 pages); each row selects 4096 ids
    spread over the whole context."""
    case = W.attn_case("long_sparse", 8211, B=1, next_n=2, Hq=8, Hkv=1, D=128, bs=16,
                       lens=[200000], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    case, sel = W.with_selection(case, 8212, 4096, window=256)
    say("long context sparse")
    d = DevAttn(case)
    import torch
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, dev(sel),
                         kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                         k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
                         softmax_scale=case.softmax_scale)
    torch.cuda.synchronize()
    ref = oracle.paged_attn_sparse(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                   case.block_table, case.context_lens, sel,
                                   **case.oracle_kwargs())
    r = compare_attn(out.cpu().numpy(), ref, case.name)
    say(f"long context sparse: max err/tol = {r:.3f}")
