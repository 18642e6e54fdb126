"""Pins for the oracle's top-k token selection (the step that turns the MQA
logits of "flashinfer.fp4_paged_mqa_logits" into the selected token ids of
"Stabilize QSA page4 order under KV relocation", Investigation and Upstream
check).

Independent references: Python's own sorted() under the stated total order
(larger logit first, NaN last, lower token id on ties); the order-free facts
any top-k must satisfy (size min(k, L); every selected value >= every
unselected one; at the threshold value the selected ids are the lowest);
k >= L selects every token; L = 0 selects none; fp16 / bf16 inputs select as
their values widened by torch do.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def logits_with_ties(seed, rows, stride, levels=7, nan_frac=0.0):
    rng = np.random.default_rng(seed)
    x = rng.integers(-levels, levels + 1, (rows, stride)).astype(np.float32) * 0.5
    x[x == 0] = np.where(rng.random((x == 0).sum()) < 0.5, -0.0, 0.0)  # both zeros
    if nan_frac:
        x[rng.random(x.shape) < nan_frac] = np.nan
    return x


def brute(x, lens, next_n, k):
    rows = len(lens) * next_n
    out = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        L = int(lens[r // next_n])
        order = sorted(range(L), key=lambda t: (math.isnan(x[r, t]),
                                                0.0 if math.isnan(x[r, t]) else -float(x[r, t]),
                                                t))
        ids = sorted(order[:k])
        out[r, :len(ids)] = ids
    return out


def pin_brute_force(lib):
    for seed, (B, N, stride, k, nan) in enumerate([(3, 2, 300, 17, 0.0), (2, 1, 1000, 100, 0.05),
                                                  (4, 3, 64, 64, 0.0), (2, 2, 50, 80, 0.1)]):
        x = logits_with_ties(seed, B * N, stride, nan_frac=nan)
        lens = np.random.default_rng(seed).integers(0, stride + 1, B).astype(np.int32)
        lens[0] = stride
        got = oracle.topk_select(x, lens, N, k, lib=lib)
        assert np.array_equal(got, brute(x, lens, N, k)), seed


def pin_order_free_facts(lib):
    B, N, stride, k = 3, 2, 500, 37
    x = logits_with_ties(11, B * N, stride, levels=3)
    lens = np.array([500, 123, 40], np.int32)
    got = oracle.topk_select(x, lens, N, k, lib=lib)
    for r in range(B * N):
        L = int(lens[r // N])
        ids = got[r][got[r] >= 0]
        assert ids.size == min(k, L) and np.all(np.diff(ids) > 0) and np.all(ids < L)
        rest = np.setdiff1d(np.arange(L), ids)
        if rest.size and ids.size:
            thr = x[r, ids].min()
            assert np.all(x[r, rest] <= thr)
            tied_out = rest[x[r, rest] == thr]
            tied_in = ids[x[r, ids] == thr]
            assert tied_out.size == 0 or tied_in.max() < tied_out.min()


def pin_edges(lib):
    x = logits_with_ties(12, 4, 30)
    lens = np.array([0, 1, 30, 7], np.int32)
    got = oracle.topk_select(x, lens, 1, 10, lib=lib)
    assert np.all(got[0] == -1)
    assert got[1, 0] == 0 and np.all(got[1, 1:] == -1)
    assert np.all(got[3, :7] == np.arange(7)) and np.all(got[3, 7:] == -1)  # k >= L
    same = np.zeros((1, 50), np.float32)
    assert np.array_equal(oracle.topk_select(same, np.array([50], np.int32), 1, 5, lib=lib)[0],
                          np.arange(5))  # all tied: the lowest ids


def pin_half_formats(lib):
    x = logits_with_ties(13, 4, 200, levels=40) * 1.37
    lens = np.array([200, 150], np.int32)
    for fmt, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        t = torch.from_numpy(x).to(dt)
        bits = t.view(torch.int16).numpy().view(np.uint16)
        got = oracle.topk_select(bits, lens, 2, 33, fmt=fmt, lib=lib)
        ref = oracle.topk_select(t.float().numpy(), lens, 2, 33, lib=lib)
        assert np.array_equal(got, ref), fmt


ALL_PINS = [pin_brute_force, pin_order_free_facts, pin_edges, pin_half_formats]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_topk_pin(orc, pin):
    pin(orc)
