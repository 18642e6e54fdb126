"""Pins for the oracle's MXFP4 paged MQA logits ("flashinfer.fp4_paged_mqa_logits"
API page: parameters q, sf_q, kv_fused, weights, context_lens, block_table,
max_context_len, out).

Independent references: per-head dot products by float64 table lookup and
einsum (exact for the workload's exponent spread, tests/brute.py), one-hot
weights (the chain then returns S_h itself, bit for bit), the fp32 recursive
summation bound for general weights, relocation invariance, the
-inf / untouched-row contract of the output, the interleaved scale-tail order
(is_kv_sf_interleaved) against the token-order cache it was rewritten from,
the rectifier variant, and the fp16 / bf16 outputs against torch's own
round-to-nearest-even conversions.
"""
import os
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


def interleave_sf_tail(case, spi=4):
    """The same cache with each block's scale tail rewritten in the interleaved
    slot order of the API page: slot k holds token (k % spi) * (bs / spi) + k / spi."""
    kv = case.kv_fused.copy()
    nb, bs = kv.shape[0], kv.shape[1]
    D = 2 * case.q.shape[-1]
    flat = kv.reshape(nb, -1)
    tail = flat[:, bs * D // 2:].reshape(nb, bs, spi).copy()
    slot_token = [(k % spi) * (bs // spi) + k // spi for k in range(bs)]
    flat[:, bs * D // 2:] = tail[:, slot_token, :].reshape(nb, -1)
    return kv, slot_token


def pin_interleaved_sf_tail(lib):
    case = small_logits(seed=11, bs=64, lens=(200, 64, 1), max_len=256)
    kv2, slot_token = interleave_sf_tail(case)
    here = os.path.dirname(os.path.abspath(__file__))
    printed = None
    for line in open(os.path.join(here, "golden", "fp4_api.txt")):
        if line.startswith("sf_interleave_slot_to_token"):
            printed = [int(x) for x in line.split("#")[0].split("=")[1].split()]
    assert slot_token[:len(printed)] == printed
    base = run(case, lib)
    got = run(dataclasses.replace(case, kv_fused=kv2), lib, sf_interleaved=True)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))
    # and reading the rewritten cache in token order is wrong (the pin has teeth)
    wrong = run(dataclasses.replace(case, kv_fused=kv2), lib)
    assert not np.array_equal(wrong.view(np.uint32), base.view(np.uint32))


def pin_relu(lib):
    case = small_logits(seed=12)
    S = brute.logits_exact(case)
    B, N, H = case.batch, case.next_n, case.num_heads
    assert any((Sb < 0).any() for Sb in S) and any((Sb > 0).any() for Sb in S)
    for h in (0, H - 1):
        w = np.zeros((B * N, H), np.float32)
        w[:, h] = 1.0
        got = run(dataclasses.replace(case, weights=w), lib, relu=True)
        for b in range(B):
            L = int(case.context_lens[b])
            for i in range(N):
                ref = np.maximum(S[b][i, :, h], 0.0)
                assert np.array_equal(got[b * N + i, :L].astype(np.float64), ref)
    got = run(case, lib, relu=True)
    w = case.weights.astype(np.float64)
    for b in range(B):
        L = int(case.context_lens[b])
        for i in range(N):
            terms = np.maximum(S[b][i], 0.0) * w[b * N + i][None, :]
            bound = H * 2.0 ** -24 * np.abs(terms).sum(1) + 1e-30
            assert np.all(np.abs(got[b * N + i, :L] - terms.sum(1)) <= bound)


def pin_output_formats(lib):
    import torch
    case = small_logits(seed=13)
    f32 = run(case, lib)
    f16 = run(case, lib, out_format="f16")
    bf16 = run(case, lib, out_format="bf16")
    t = torch.from_numpy(f32)
    assert np.array_equal(f16.view(np.uint16), t.to(torch.float16).numpy().view(np.uint16))
    assert np.array_equal(bf16, t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert (bf16[0, int(case.context_lens[0]):case.max_context_len] == 0xFF80).all()  # -inf


def epi_chain_numpy(S, w, epi):
    """The reduced-precision head chain written with numpy and torch casts: the
    weight and the dot rounded to the epilogue type (torch's round to nearest
    even), an fp32 fused multiply-add (exact product and sum in float64, one
    rounding to float32, which equals fmaf for float32 operands), then the
    running value rounded to the epilogue type."""
    import torch
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[epi]
    rnd = lambda x: torch.from_numpy(np.asarray(x, np.float32)).to(dt).float().numpy()
    acc = np.zeros(S.shape[0], np.float32)
    ws, ss = rnd(w), rnd(S.astype(np.float32))
    for h in range(S.shape[1]):
        fma = (ws[h].astype(np.float64) * ss[:, h].astype(np.float64) +
               acc.astype(np.float64)).astype(np.float32)
        acc = rnd(fma)
    return acc


def pin_epilogue_types(lib):
    """fp16 / bf16 epilogues (the reading stated at epi_step in oracle.c)
    against the numpy/torch chain on the exact dots, bit for bit; and they are
    not the fp32 result (the pin has teeth)."""
    case = small_logits(seed=14)
    S = brute.logits_exact(case)
    f32 = run(case, lib)
    for epi in ("f16", "bf16"):
        got = run(case, lib, epi_format=epi)
        for b in range(case.batch):
            L = int(case.context_lens[b])
            for i in range(case.next_n):
                r = b * case.next_n + i
                ref = epi_chain_numpy(S[b][i], case.weights[r], epi)
                assert np.array_equal(got[r, :L].view(np.uint32), ref.view(np.uint32)), epi
                assert np.all(got[r, L:case.max_context_len] == -np.inf)
        assert not np.array_equal(got.view(np.uint32), f32.view(np.uint32))


ALL_PINS = [pin_one_hot_weights_exact, pin_weighted_sum_bound, pin_tail_and_rows, pin_relocation,
            pin_interleaved_sf_tail, pin_relu, pin_output_formats, pin_epilogue_types]


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
