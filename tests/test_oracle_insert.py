"""Pins for the oracle's KV insert (the KV-only insert path of "DeepSeek-V4.1
Q pad + fused KV insert": rows beyond the slots, or with no slot, are
skipped; the test compares cache bytes with rtol=0, atol=0 into a NaN-filled
destination).

Independent references: torch's float8_e4m3fn cast for E4M3 codes, numpy
rint/clip for INT8/INT4, exact round trips of every code, bit copies for fp16.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import brute


def run(case, lib):
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    oracle.kv_insert(kc, vc, case.kv_kind, case.k, case.v, case.slot_mapping,
                     k_scale=case.k_scale, k_scale_mode=case.scale_mode, v_scale=case.v_scale,
                     v_scale_mode=case.scale_mode, block_size=case.block_size,
                     in_is_bf16=case.in_bf16, lib=lib)
    return kc, vc


def expected_codes(x, scale, kind, mode):
    """Reference codes [T, Hkv, D] via library routines."""
    x = x.astype(np.float32)
    if mode == W.SCALE_PER_TENSOR:
        y = x / np.float32(scale[0])
    elif mode == W.SCALE_PER_CHANNEL:
        y = x / scale.astype(np.float32)[None]
    else:
        y = x
    if kind == W.KV_E4M3:
        return torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
    lim = 127 if kind == W.KV_INT8 else 7
    return np.clip(np.rint(y), -lim, lim).astype(np.int8)


def check_case(case, lib):
    kc, vc = run(case, lib)
    T = case.k.shape[0]
    bs = case.block_size
    written = np.zeros(kc.shape[:2], bool)
    for cache, x, scale in ((kc, case.k, case.k_scale), (vc, case.v, case.v_scale)):
        codes = None if case.kv_kind in (W.KV_F16, W.KV_BF16) else expected_codes(
            case.values(x), scale, case.kv_kind, case.scale_mode)
        for i in range(T):
            if i >= case.slot_mapping.shape[0] or case.slot_mapping[i] < 0:
                continue
            s = int(case.slot_mapping[i])
            blk, off = s // bs, s % bs
            if blk >= kc.shape[0]:
                continue  # past the cache: skipped
            written[blk, off] = True
            row = cache[blk, off]
            if case.kv_kind in (W.KV_F16, W.KV_BF16):
                assert np.array_equal(row.view(np.uint16), x[i].view(np.uint16))
            elif case.kv_kind == W.KV_INT4:
                dec = brute.decode_cache(row[None, None], W.KV_INT4, x.shape[-1])[0, 0]
                assert np.array_equal(dec.astype(np.int8), codes[i])
            elif case.kv_kind == W.KV_INT8:
                assert np.array_equal(row.view(np.int8), codes[i])
            else:
                assert np.array_equal(row, codes[i])
    assert np.all(kc[~written] == 0xFF) and np.all(vc[~written] == 0xFF)


def pin_insert_vs_library(lib):
    for kind, mode in ((W.KV_E4M3, W.SCALE_PER_TENSOR), (W.KV_E4M3, W.SCALE_PER_CHANNEL),
                       (W.KV_INT8, W.SCALE_PER_TENSOR), (W.KV_INT8, W.SCALE_PER_CHANNEL),
                       (W.KV_INT4, W.SCALE_PER_TENSOR), (W.KV_INT4, W.SCALE_PER_CHANNEL),
                       (W.KV_F16, W.SCALE_NONE)):
        case = W.insert_case(17, T=37, Hkv=2, D=32, bs=8, kv_kind=kind, scale_mode=mode,
                             slotless_tail=5, neg_slots=3, value_scale=3.0)
        check_case(case, lib)


def pin_round_trip_every_code(lib):
    """Values code * 2^-3 insert back to exactly the code they came from."""
    s = np.array([0.125], np.float32)
    for kind, codes in ((W.KV_E4M3, [c for c in range(256) if c not in (0x7F, 0xFF)]),
                        (W.KV_INT8, list(range(-127, 128))), (W.KV_INT4, list(range(-7, 8)))):
        n = len(codes)
        D = 16
        T = -(-n // D)
        if kind == W.KV_E4M3:
            vals = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
        else:
            vals = np.array(codes, np.float32)
        x = np.zeros(T * D, np.float32)
        x[:n] = vals * s[0]
        x = x.reshape(T, 1, D).astype(np.float16)
        assert np.array_equal(x.astype(np.float32).reshape(-1)[:n], vals * s[0])
        case = W.InsertCase(k=x, v=x, slot_mapping=np.arange(8, 8 + T, dtype=np.int64),
                            num_blocks=T // 8 + 2, block_size=8, kv_kind=kind, k_scale=s,
                            v_scale=s, scale_mode=W.SCALE_PER_TENSOR,
                            k_cache=np.full((T // 8 + 2, 8, 1, W.row_bytes(kind, D)), 0xFF,
                                            np.uint8),
                            v_cache=np.full((T // 8 + 2, 8, 1, W.row_bytes(kind, D)), 0xFF,
                                            np.uint8))
        kc, _ = run(case, lib)
        rows = kc.reshape(-1, 1, W.row_bytes(kind, D))[8:8 + T]
        if kind == W.KV_E4M3:
            got = rows.reshape(-1)[:n]
            assert np.array_equal(got, np.array(codes, np.uint8))
        else:
            got = brute.decode_cache(rows[:, None], kind, D).reshape(-1)[:n]
            assert np.array_equal(got.astype(np.int64), np.array(codes))


def pin_bf16_input_and_cache(lib):
    """bf16 input rows: quantized from their bf16 values (torch's own bf16),
    or copied bit for bit into a BF16 cache."""
    for kind, mode in ((W.KV_E4M3, W.SCALE_PER_TENSOR), (W.KV_INT8, W.SCALE_PER_CHANNEL),
                       (W.KV_INT4, W.SCALE_PER_TENSOR), (W.KV_BF16, W.SCALE_NONE)):
        case = W.insert_case(19, T=29, Hkv=2, D=32, bs=8, kv_kind=kind, scale_mode=mode,
                             slotless_tail=3, neg_slots=2, value_scale=2.0, in_dtype="bf16")
        check_case(case, lib)


def pin_slot_past_cache_skipped(lib):
    """A slot at or past num_blocks * block_size is skipped: the cache equals
    the insert of the other rows alone."""
    case = W.insert_case(23, T=40, Hkv=1, D=32, bs=8, kv_kind=W.KV_INT8,
                         scale_mode=W.SCALE_PER_TENSOR, oob_slots=3)
    bad = case.slot_mapping >= case.num_blocks * case.block_size
    assert bad.sum() == 3
    kc, vc = run(case, lib)
    import dataclasses
    clean = dataclasses.replace(case, slot_mapping=np.where(bad, -1, case.slot_mapping))
    kc2, vc2 = run(clean, lib)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)
    check_case(case, lib)


ALL_PINS = [pin_insert_vs_library, pin_round_trip_every_code, pin_bf16_input_and_cache,
            pin_slot_past_cache_skipped]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_insert_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("T", [17, 1024, 2049])
@pytest.mark.parametrize("tail", [0, 5])
def test_insert_token_counts(orc, T, tail):
    """Token counts and slotless rows of the pages' insert test."""
    case = W.insert_case(T + tail, T=T, Hkv=1, D=64, bs=16, kv_kind=W.KV_E4M3,
                         scale_mode=W.SCALE_PER_TENSOR, slotless_tail=tail)
    check_case(case, orc)
