"""Pins for the oracle's scalar codecs, against library conversions (torch's
float8 / bfloat16 casts, numpy's float16) and the values the pages print.

Pages: "Stop grouped-page4 null-block padding from leaking E4M3 NaN" (Root
cause: E4M3 bytes 0x7F/0xFF decode to NaN, fp16 0x7e00); the fp8 decode
workload's quantization scale max|x|/448 (448 = largest finite E4M3);
"Normalize the PER_CHANNEL K scale ..." (Description: INT4 scale max|K|/7,
INT8 max|K|/127, "roughly 18x").
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f32(codes, orc)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert np.array_equal(ours[~nan_ours].view(np.uint32), ref[~nan_ours].view(np.uint32))


def test_e4m3_pages_values(orc):
    # NaN codes named by the pages, and the 448 maximum of the fp8 decode recipe
    assert math.isnan(orc.orc_e4m3_to_f32(0x7F)) and math.isnan(orc.orc_e4m3_to_f32(0xFF))
    finite = [orc.orc_e4m3_to_f32(c) for c in range(256) if c not in (0x7F, 0xFF)]
    assert max(finite) == 448.0 and min(finite) == -448.0
    assert orc.orc_e4m3_to_f32(0x7E) == 448.0
    # the smallest subnormal is 2^-9
    assert orc.orc_e4m3_to_f32(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_sweep(orc):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-500, 500, 4000), rng.standard_normal(4000) * 3,
        rng.standard_normal(2000) * 1e-2, np.array([0.0, -0.0, 448.0, -448.0, 1e9, -1e9]),
    ]).astype(np.float32)
    # exact midpoints between consecutive finite codes exercise ties-to-even
    vals = oracle.e4m3_to_f32(np.arange(0, 0x7E, dtype=np.uint8), orc).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = oracle.f32_to_e4m3(x, orc)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_decode_identity(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert orc.orc_f32_to_e4m3(orc.orc_e4m3_to_f32(c)) == c


def test_f16_decode_matches_numpy_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = np.array([orc.orc_f16_to_f32(int(c)) for c in codes], np.float32)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert orc.orc_f16_to_f32(0x7E00) != orc.orc_f16_to_f32(0x7E00)  # fp16 0x7e00 is NaN


def test_f64_to_f16_matches_numpy(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-20, 12, 20000)),
        np.array([65504.0, 65519.999, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0001, 3 * 2.0 ** -26, 6.1e-5, 0.0, -0.0]),
    ])
    ours = oracle.f64_to_f16(x, orc)
    ref = x.astype(np.float16)
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))


def test_bf16_codecs_match_torch(orc):
    codes = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = np.array([orc.orc_bf16_to_f32(int(c)) for c in codes], np.float32)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    x = (np.random.default_rng(5).standard_normal(5000) * 100).astype(np.float32)
    ours = np.array([orc.orc_f32_to_bf16(float(v)) for v in x], np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_int_round_clamp(orc):
    y = np.array([2.5, 3.5, -2.5, -3.5, 0.49999997, 126.5, 127.4, 200.0, -200.0, 6.5, 7.5, -7.6],
                 np.float32)
    for lim in (127, 7):
        ours = [orc.orc_round_clamp(float(v), lim) for v in y]
        ref = np.clip(np.rint(y), -lim, lim).astype(int).tolist()
        assert ours == ref
    assert orc.orc_round_clamp(2.5, 127) == 2 and orc.orc_round_clamp(3.5, 127) == 4


def test_int4_nibble_sign_extension(orc):
    for n in range(16):
        ref = int(np.array([n << 4], np.uint8).view(np.int8)[0]) >> 4
        assert orc.orc_int4_value(n) == ref


def test_int4_int8_scale_ratio():
    # "roughly 18x": INT4's max|K|/7 against INT8's max|K|/127 for identical data
    assert abs(127 / 7 - 18.14) < 0.01


def test_e2m1_decode_table(orc):
    # OCP MX E2M1 magnitudes for codes 0..7; bit 3 is the sign
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = orc.orc_e2m1_to_f32(c)
        mag = table[c & 7]
        assert v == (-mag if c & 8 else mag)
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def test_ue8m0_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([orc.orc_ue8m0_to_f32(int(c)) for c in codes], np.float32)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy()
    assert math.isnan(ours[255]) and math.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


@pytest.mark.parametrize("kind", [oracle.KV_E4M3, oracle.KV_INT8, oracle.KV_INT4, oracle.KV_F16])
@pytest.mark.parametrize("mode", [oracle.SCALE_NONE, oracle.SCALE_PER_TENSOR,
                                  oracle.SCALE_PER_CHANNEL])
def test_dequantize_is_code_times_scale(orc, kind, mode):
    rng = np.random.default_rng(11)
    n, ch = 512, 64
    if kind == oracle.KV_F16:
        codes = rng.standard_normal(n).astype(np.float16).view(np.uint8)
        vals = codes.view(np.float16).astype(np.float32)
    elif kind == oracle.KV_INT4:
        codes = rng.integers(0, 256, n // 2, dtype=np.uint8)
        nib = np.stack([codes & 15, codes >> 4], -1).reshape(-1).astype(np.int8)
        vals = np.where(nib >= 8, nib - 16, nib).astype(np.float32)
    elif kind == oracle.KV_INT8:
        codes = rng.integers(0, 256, n, dtype=np.uint8)
        vals = codes.view(np.int8).astype(np.float32)
    else:
        codes = rng.integers(0, 256, n, dtype=np.uint8)
        vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    scale = np.exp(rng.uniform(-3, 3, ch)).astype(np.float32)
    out = oracle.dequantize(kind, codes, n, scale, mode, ch, orc)
    if mode == oracle.SCALE_NONE:
        ref = vals
    elif mode == oracle.SCALE_PER_TENSOR:
        ref = vals * scale[0]
    else:
        ref = vals * np.tile(scale, n // ch)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(out[~nan], ref[~nan])
