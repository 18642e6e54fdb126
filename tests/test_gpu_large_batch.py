"""Large batches: 8192 short decode sequences (every workgroup's range scan
walks all 8192 lengths, the merge launches one workgroup per sequence and KV
head), 1024 logits rows, and top-k over 2048 rows, against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import compare_attn, dev, run_attn, say

pytestmark = pytest.mark.gpu


def test_decode_8192_sequences(pa):
    rng = np.random.default_rng(8301)
    lens = rng.integers(0, 70, 8192)
    case = W.attn_case("batch_8192", 8301, B=8192, next_n=1, Hq=4, Hkv=1, D=128, bs=16,
                       lens=list(lens), kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR,
                       max_context_len=80)
    say("decode B=8192")
    got = run_attn(pa, case)
    ref = oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                            case.context_lens, **case.oracle_kwargs())
    r = compare_attn(got, ref, case.name)
    say(f"decode B=8192: max err/tol = {r:.3f}")


def test_logits_and_topk_many_rows(pa):
    """512 sequences x 2 query rows of logits (bit-exact), then top-k 64 over
    their 1024 rows (bit-exact), and top-k over 2048 rows of random logits."""
    rng = np.random.default_rng(8311)
    lens = rng.integers(1, 600, 512).astype(np.int32)
    lg = W.logits_case("rows_1024", 8311, B=512, next_n=2, H=16, D=128, bs=64, lens=lens,
                       max_context_len=640)
    say("logits 1024 rows")
    got = pa.paged_mqa_logits(dev(lg.q), dev(lg.sf_q), dev(lg.kv_fused), dev(lg.weights),
                              dev(lens), dev(lg.block_table), lg.max_context_len)
    ref = oracle.mqa_logits(lg.q, lg.sf_q, lg.kv_fused, lg.weights, lens, lg.block_table,
                            lg.max_context_len)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    say("top-k over 1024 logits rows")
    sel = pa.topk_select(got, dev(lens), 2, 64)
    assert np.array_equal(sel.cpu().numpy(), oracle.topk_select(ref, lens, 2, 64))
    x = rng.standard_normal((2048, 3000)).astype(np.float32)
    lens2 = rng.integers(0, 3001, 1024).astype(np.int32)
    say("top-k over 2048 rows")
    sel2 = pa.topk_select(dev(x), dev(lens2), 2, 300)
    assert np.array_equal(sel2.cpu().numpy(), oracle.topk_select(x, lens2, 2, 300))
