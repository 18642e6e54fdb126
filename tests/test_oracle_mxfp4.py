"""Pins for the oracle's MXFP4 insert: E2M1 codes with one UE8M0 scale byte per
32 values, written into the kv_fused block layout of the
"flashinfer.fp4_paged_mqa_logits" API page (kv_fused, is_kv_sf_interleaved).

The pages print no quantizer; the oracle takes the OCP Microscaling rule
(scale 2^(floor(log2 amax) - 2), nearest-even E2M1 codes saturating at 6).
Independent references: the E2M1 value table (brute.E2M1) for the round trip
of all 16 codes; the textbook ties of the E2M1 grid and saturation; Python's
math.floor(math.log2(.)) for the scale byte; groups built from representable
values, which must come back exactly; a per-element error bound on random
rows; the logits reference reading the inserted cache (interleaved and token
order give the same logits); and the skip rule for rows without a slot.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import brute


def decode_fused(kv, D=128, sf_interleaved=False):
    """Dequantized [num_blocks, bs, D] float64 values of a kv_fused cache, from
    the E2M1 table and 2^(byte - 127), reading the scale slot of each token."""
    nb, bs = kv.shape[0], kv.shape[1]
    flat = kv.reshape(nb, -1)
    data = flat[:, :bs * D // 2].reshape(nb, bs, D // 2)
    sf = flat[:, bs * D // 2:].reshape(nb, bs, D // 32)
    if sf_interleaved:
        slot_of = {(k % 4) * (bs // 4) + k // 4: k for k in range(bs)}
        sf = sf[:, [slot_of[t] for t in range(bs)], :]
    nib = np.stack([data & 15, data >> 4], -1).reshape(nb, bs, D)
    return brute.E2M1[nib] * np.ldexp(1.0, np.repeat(sf.astype(np.int64), 32, -1) - 127)


def pin_e2m1_round_trip(lib):
    codes = np.arange(16, dtype=np.uint8)
    vals = brute.E2M1[codes].astype(np.float32)
    vals[8] = -0.0
    assert np.array_equal(oracle.f32_to_e2m1(vals, lib), codes)


def pin_e2m1_ties_and_saturation(lib):
    # midpoints of the E2M1 grid go to the code with an even mantissa bit
    y = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 6.0, 6.5, 1e9, 0.26, 4.9]
    want = [0, 2, 2, 4, 4, 6, 6, 8, 14, 7, 7, 7, 1, 6]
    assert oracle.f32_to_e2m1(y, lib).tolist() == want


def pin_scale_byte(lib):
    rng = np.random.default_rng(21)
    amax = np.concatenate([np.exp2(rng.uniform(-60, 60, 500)), [1.0, 6.0, 0.75, 2.0 ** -130,
                                                                  3.0e38]]).astype(np.float32)
    got = oracle.mx_scale_byte(amax, lib)
    want = [min(254, max(0, math.floor(math.log2(float(a))) - 2 + 127)) for a in amax]
    assert got.tolist() == want
    assert int(oracle.mx_scale_byte([0.0], lib)[0]) == 0


def representable_case(seed):
    """Rows whose every 32-group is E2M1 codes times 2^(B-127) with one element
    of magnitude 4 or 6: the group's scale byte must be B and the values exact."""
    rng = np.random.default_rng(seed)
    T, D = 40, 128
    codes = rng.integers(0, 16, (T, D))
    top = rng.choice([6, 7], (T, D // 32))  # magnitude 4 or 6
    codes.reshape(T, D // 32, 32)[:, :, 0] = top | (rng.integers(0, 2, (T, D // 32)) * 8)
    B = rng.integers(118, 136, (T, D // 32))
    x = brute.E2M1[codes] * np.ldexp(1.0, np.repeat(B, 32, -1) - 127)
    return x, codes, B


def pin_representable_groups_exact(lib):
    x, codes, B = representable_case(22)
    T, D = x.shape
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.float16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.float16).astype(np.float64), x)  # exact in fp16
    kv = np.full((T // 64 + 3, 64, 1, 68), 0xFF, np.uint8)
    slots = np.arange(64, 64 + T, dtype=np.int64)
    oracle.mxfp4_insert(kv, bits.view(np.uint16), slots, lib=lib)
    deq = decode_fused(kv).reshape(-1, D)[64:64 + T]
    assert np.array_equal(deq, x)
    sf = kv.reshape(kv.shape[0], -1)[:, 64 * 64:].reshape(-1, D // 32)[64:64 + T]
    assert np.array_equal(sf.astype(np.int64), B)


def pin_error_bound(lib):
    case = W.mxfp4_insert_case(23, T=96, in_dtype="bf16")
    kv = case.kv_fused
    oracle.mxfp4_insert(kv, case.k_bits, case.slot_mapping, in_dtype="bf16", lib=lib)
    x = torch.from_numpy(case.k_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    deq = decode_fused(kv)
    for i, s in enumerate(case.slot_mapping):
        got = deq[s // 64, s % 64]
        g = x[i].reshape(-1, 32)
        amax = np.abs(g).max(1, keepdims=True)
        X = np.where(amax > 0, np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2), 0)
        y = np.abs(g) / np.where(X > 0, X, 1)
        half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
        bound = np.maximum(half_step, y - 6.0) * X  # rounding, or saturation above 6
        assert np.all(np.abs(got.reshape(-1, 32) - g) <= bound + 1e-300), i


def pin_interleaved_insert_reads_back(lib):
    base = W.mxfp4_insert_case(24, T=150, slotless_tail=4, neg_slots=3)
    kv_t = base.kv_fused.copy()
    kv_i = base.kv_fused.copy()
    oracle.mxfp4_insert(kv_t, base.k_bits, base.slot_mapping, lib=lib)
    oracle.mxfp4_insert(kv_i, base.k_bits, base.slot_mapping, sf_interleaved=True, lib=lib)
    assert not np.array_equal(kv_t, kv_i)
    assert np.array_equal(decode_fused(kv_t), decode_fused(kv_i, sf_interleaved=True))
    # the logits reference reads both caches to the same logits
    rng = np.random.default_rng(25)
    used = sorted({int(s) // 64 for s in base.slot_mapping if s >= 0})
    bt = np.array([used], np.int32)
    L = 64 * len(used)
    q = rng.integers(0, 256, (1, 1, 16, 64), dtype=np.uint8)
    sfq = rng.integers(0x7A000000, 0x7A7F7F7F, (1, 1, 16), dtype=np.int64).astype(np.int32)
    w = rng.standard_normal((1, 16)).astype(np.float32)
    cl = np.array([L], np.int32)
    a = oracle.mqa_logits(q, sfq, kv_t, w, cl, bt, L, lib=lib)
    b = oracle.mqa_logits(q, sfq, kv_i, w, cl, bt, L, sf_interleaved=True, lib=lib)
    assert np.array_equal(np.nan_to_num(a).view(np.uint32), np.nan_to_num(b).view(np.uint32))


def pin_slotless_rows_untouched(lib):
    case = W.mxfp4_insert_case(26, T=70, slotless_tail=5, neg_slots=4)
    kv = case.kv_fused.copy()
    oracle.mxfp4_insert(kv, case.k_bits, case.slot_mapping, lib=lib)
    written = np.zeros(kv.shape[:2], bool)
    for s in case.slot_mapping:
        if s >= 0:
            written[s // 64, s % 64] = True
    flat = kv.reshape(kv.shape[0], -1)
    data = flat[:, :64 * 64].reshape(kv.shape[0], 64, 64)
    sf = flat[:, 64 * 64:].reshape(kv.shape[0], 64, 4)
    assert (data[~written] == 0xFF).all() and (sf[~written] == 0xFF).all()
    assert (sf[written] != 0xFF).all()
    assert int((case.slot_mapping >= 0).sum()) == int(written.sum())


ALL_PINS = [pin_e2m1_round_trip, pin_e2m1_ties_and_saturation, pin_scale_byte,
            pin_representable_groups_exact, pin_error_bound, pin_interleaved_insert_reads_back,
            pin_slotless_rows_untouched]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_mxfp4_pin(orc, pin):
    pin(orc)
