"""Pins for the oracle's MXFP4 paged MQA logits ("flashinfer.fp4_paged_mqa_logits"
API page: parameters q, sf_q, kv_fused, weights, context_lens, block_table,
max_context_len, out).

Independent references: per-head dot products by float64 table lookup and
einsum (exact for the workload's exponent spread, tests/brute.py), one-hot
weights (the chain then returns S_h itself, bit for bit), the fp32 recursive
summation bound for general weights, relocation invariance, and the
-inf / untouched-row contract of the output.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests import brute


def small_logits(seed=3, B=3, N=2, H=8, bs=16, lens=(37, 64, 1), max_len=80):
    return W.logits_case("small", seed, B=B, next_n=N, H=H, D=128, bs=bs, lens=list(lens),
                         max_context_len=max_len)


def run(case, lib, **kw):
    return oracle.mqa_logits(case.q, case.sf_q, case.kv_fused, case.weights, case.context_lens,
                             case.block_table, case.max_context_len, lib=lib, **kw)


def pin_one_hot_weights_exact(lib):
    case = small_logits()
    S = brute.logits_exact(case)
    B, N, H = case.batch, case.next_n, case.num_heads
    for h in (0, 3, H - 1):
        w = np.zeros((B * N, H), np.float32)
        w[:, h] = 1.0
        got = run(dataclasses.replace(case, weights=w), lib)
        for b in range(B):
            L = int(case.context_lens[b])
            for i in range(N):
                ref = S[b][i, :, h]
                assert np.array_equal(got[b * N + i, :L].astype(np.float64), ref)


def pin_weighted_sum_bound(lib):
    case = small_logits(seed=4)
    S = brute.logits_exact(case)
    got = run(case, lib)
    B, N, H = case.batch, case.next_n, case.num_heads
    w = case.weights.astype(np.float64)
    for b in range(B):
        L = int(case.context_lens[b])
        for i in range(N):
            terms = S[b][i] * w[b * N + i][None, :]  # [L, H]
            ref = terms.sum(1)
            bound = H * 2.0 ** -24 * np.abs(terms).sum(1) + 1e-30
            assert np.all(np.abs(got[b * N + i, :L] - ref) <= bound)


def pin_tail_and_rows(lib):
    case = small_logits(seed=5)
    rows, stride = case.batch * case.next_n + 3, case.max_context_len + 7
    got = run(case, lib, out_rows=rows, out_row_stride=stride)
    for b in range(case.batch):
        L = int(case.context_lens[b])
        for i in range(case.next_n):
            r = b * case.next_n + i
            assert np.isfinite(got[r, :L]).all()
            assert np.all(got[r, L:case.max_context_len] == -np.inf)
            assert np.isnan(got[r, case.max_context_len:]).all()  # beyond max_context_len: untouched
    assert np.isnan(got[case.batch * case.next_n:]).all()  # extra rows untouched


def pin_relocation(lib):
    case = small_logits(seed=6)
    base = run(case, lib)
    rng = np.random.default_rng(8)
    nb = case.kv_fused.shape[0]
    perm = rng.permutation(np.arange(1, nb))
    remap = np.zeros(nb, np.int64)
    remap[1:] = perm
    kv2 = rng.integers(0, 256, case.kv_fused.shape, dtype=np.uint8)
    kv2[0] = case.kv_fused[0]
    kv2[remap[1:]] = case.kv_fused[1:]
    bt2 = np.where(case.block_table > 0, remap[case.block_table], 0).astype(np.int32)
    got = run(dataclasses.replace(case, kv_fused=kv2, block_table=bt2), lib)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


ALL_PINS = [pin_one_hot_weights_exact, pin_weighted_sum_bound, pin_tail_and_rows, pin_relocation]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_logits_pin(orc, pin):
    pin(orc)


def test_table_width_rule(orc):
    """context_len = 257 with block_size = 64 needs round_up(257, 128) / 64 = 6
    columns (API page, block_table parameter); the padding column may be any
    valid index and is never dereferenced by the reference."""
    case = W.logits_case("w", 9, B=1, next_n=1, H=4, D=128, bs=64, lens=[257],
                         max_context_len=257)
    assert case.block_table.shape[1] == 6
    assert (-(-257 // 128) * 128) // 64 == 6 and -(-257 // 64) == 5
    base = run(case, orc)
    bt = case.block_table.copy()
    bt[0, 5] = 12345678  # never read: past ceil(257 / 64) = 5 blocks
    assert np.array_equal(run(dataclasses.replace(case, block_table=bt), orc).view(np.uint32),
                          base.view(np.uint32))


def test_kv_row_bytes():
    # kv_row_bytes = head_dim/2 + head_dim/sf_vec_size: 68 at D = 128, 4352 B per 64-token block
    case = small_logits(bs=64, lens=(64, 10, 5))
    assert case.kv_fused.shape[-1] == 68
    assert case.kv_fused.shape[1] * case.kv_fused.shape[-1] == 4352


def test_exponent_spread_keeps_dots_exact():
    """With UE8M0 exponents in [125, 129] the per-group sums span at most
    8 + 13 bits, so every S_h is exactly representable in fp32."""
    case = small_logits(seed=10)
    for Sb in brute.logits_exact(case):
        assert np.array_equal(Sb.astype(np.float32).astype(np.float64), Sb)
