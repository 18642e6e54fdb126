"""GPU parity of pa_topk_select (the top-k that turns MQA logits into each
query row's token set, "Stabilize QSA page4 order under KV relocation",
Investigation and Upstream check) against the oracle, bit for bit (index
work), and the whole chain paged_mqa_logits -> pa_topk_select ->
paged_attn_sparse against the oracle's chain."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DevAttn, compare_attn_conditioned, dev, log_parity, say
from tests.test_oracle_topk import logits_with_ties

pytestmark = pytest.mark.gpu


def cases():
    """(name, logits float32 [rows, stride], lens, next_n, k)"""
    out = []
    rng = np.random.default_rng(61)
    x = logits_with_ties(61, 8, 5000, levels=20)
    out.append(("ties", x, np.array([5000, 4999, 3, 0], np.int32), 2, 2048))
    x = logits_with_ties(62, 6, 3000, levels=3, nan_frac=0.02)
    out.append(("few_levels_nan", x, np.array([3000, 1024, 1025], np.int32), 2, 1024))
    x = rng.standard_normal((3, 700)).astype(np.float32)
    out.append(("k1", x, np.array([700, 1, 2], np.int32), 1, 1))
    x = rng.standard_normal((4, 33000)).astype(np.float32)
    out.append(("long", x, np.array([33000, 32768], np.int32), 2, 2048))
    x = np.zeros((2, 1500), np.float32)
    x[1, ::2] = -0.0
    out.append(("all_equal_signed_zeros", x, np.array([1500, 1499], np.int32), 1, 77))
    # a row stride that is not a multiple of 4 (the keys are read one at a time)
    x = rng.standard_normal((4, 2999)).astype(np.float32)
    out.append(("odd_stride", x, np.array([2999, 2500], np.int32), 2, 512))
    # full-length rows of widely spread values (the candidate route)
    x = (rng.standard_normal((3, 32768)) * 5000).astype(np.float32)
    out.append(("wide_full", x, np.array([32768, 32767, 20001], np.int32), 1, 2048))
    # long rows of one value: more keys share the pivot bins than the
    # candidate lists hold (the radix route)
    x = np.zeros((2, 20000), np.float32)
    out.append(("all_equal_long", x, np.array([20000, 19000], np.int32), 1, 100))
    out.append(("sample_miss", sample_miss_row(20000), np.array([20000], np.int32), 1, 2048))
    # k one below the row length, and k at half of it
    x = rng.standard_normal((2, 5000)).astype(np.float32)
    out.append(("k_near_L", x, np.array([5000, 5000], np.int32), 1, 4999))
    out.append(("k_half", x.copy(), np.array([5000, 4000], np.int32), 1, 2500))
    # half of a long row NaN: the k-th key may be NaN's (key 0)
    x = rng.standard_normal((2, 20000)).astype(np.float32)
    x[:, rng.random(20000) < 0.5] = np.nan
    out.append(("nan_half", x, np.array([20000, 20000], np.int32), 1, 12000))
    # the k-th value is 0 with +0 and -0 mixed among many zeros
    x = np.concatenate([np.abs(rng.standard_normal((2, 3000))), np.zeros((2, 9000)),
                        -np.abs(rng.standard_normal((2, 3000)))], axis=1).astype(np.float32)
    x[:, 3000:12000:2] = -0.0
    x = x[:, rng.permutation(15000)].copy()
    out.append(("zero_threshold", x, np.array([15000, 14999], np.int32), 1, 7000))
    # values on a few levels spread over the whole row (ties at T across waves)
    x = rng.integers(-3, 4, (2, 30000)).astype(np.float32) * 0.25
    out.append(("few_levels_long", x, np.array([30000, 29999], np.int32), 1, 9000))
    return out


def sample_miss_row(L):
    """One row whose large values sit only at ids the pivot route does not
    sample: wave w of 16 owns ids [w c, (w + 1) c), c = round_up(ceil(L / 16),
    256), and samples offset o = 256 u + 4 l + e when u and lane l have the
    same parity and e = (l >> 4) & 3. The sample sees only small values, so
    its pivots put almost every key above T and the row takes the radix
    route."""
    rng = np.random.default_rng(67)
    c = ((L + 15) // 16 + 255) // 256 * 256
    ids = np.arange(L)
    o = ids % c
    u, l, e = o // 256, (o % 256) // 4, o % 4
    sampled = ((u & 1) == (l & 1)) & (e == ((l >> 4) & 3))
    x = np.where(sampled, rng.random(L), 10.0 + rng.random(L)).astype(np.float32)
    return x.reshape(1, L).copy()


@pytest.mark.parametrize("idx", range(14))
@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_topk_bit_exact(pa, idx, fmt):
    name, x, lens, N, k = cases()[idx]
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[fmt]
    t = torch.from_numpy(x).to(dt)
    say(f"topk {name} fmt={fmt} k={k}")
    got = pa.topk_select(t.cuda(), dev(lens), N, k).cpu().numpy()
    src = x if fmt == "f32" else t.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.topk_select(src, lens, N, k, fmt=fmt)
    assert np.array_equal(got, ref), name


def test_topk_full_logits_workload(pa):
    """k = 2048 over the logits kernel's output at the full logits workload."""
    case = W.mxfp4_logits()
    say("topk over the full logits workload")
    logits = pa.paged_mqa_logits(dev(case.q), dev(case.sf_q), dev(case.kv_fused),
                                 dev(case.weights), dev(case.context_lens),
                                 dev(case.block_table), case.max_context_len)
    sel = pa.topk_select(logits, dev(case.context_lens), case.next_n, 2048)
    torch.cuda.synchronize()
    ref = oracle.topk_select(logits.cpu().numpy(), case.context_lens, case.next_n, 2048)
    assert np.array_equal(sel.cpu().numpy(), ref)


def test_logits_topk_sparse_chain(pa):
    """Indexer logits over an MXFP4 cache -> top-k ids -> sparse attention over
    an E4M3 cache of the same sequences: the logits and the ids equal the
    oracle's bit for bit, the attention is within tolerance of the oracle
    chain's."""
    B, N, k = 4, 2, 256
    lens = np.array([2900, 700, 257, 40], np.int32)
    lg = W.logits_case("chain_idx", 6201, B=B, next_n=N, H=64, D=128, bs=64, lens=lens,
                       max_context_len=3072)
    at = W.attn_case("chain_attn", 6202, B=B, next_n=N, Hq=16, Hkv=2, D=128, bs=32, lens=lens,
                     kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR, max_context_len=3072)
    say("chain: logits")
    logits = pa.paged_mqa_logits(dev(lg.q), dev(lg.sf_q), dev(lg.kv_fused), dev(lg.weights),
                                 dev(lg.context_lens), dev(lg.block_table), lg.max_context_len)
    sel = pa.topk_select(logits, dev(lg.context_lens), N, k)
    d = DevAttn(at)
    out = torch.full(at.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    say("chain: sparse attention")
    pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, at.max_context_len,
                         sel.view(B, N, k), kv_kind=at.kv_kind, k_scale=d.ks, v_scale=d.vs)
    torch.cuda.synchronize()
    lo = oracle.mqa_logits(lg.q, lg.sf_q, lg.kv_fused, lg.weights, lg.context_lens,
                           lg.block_table, lg.max_context_len)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), lo.view(np.uint32))
    so = oracle.topk_select(lo, lg.context_lens, N, k)
    assert np.array_equal(sel.cpu().numpy(), so)
    ref, cond, vr = oracle.paged_attn_sparse(at.q, at.k_cache, at.v_cache, at.kv_kind,
                                             at.block_table, at.context_lens,
                                             so.reshape(B, N, k), conditioning=True,
                                             **at.oracle_kwargs())
    st = compare_attn_conditioned(out.cpu().numpy(), ref, cond, vr, "chain")
    say(f"chain: {st}")
    log_parity({"test": "chain", "case": "logits_topk_sparse", **st})
