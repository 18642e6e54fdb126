"""GPU bit-exactness of the cache codecs (pa_dequantize, the decoder the
attention kernel uses) and of kv_insert, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [W.KV_E4M3, W.KV_INT8, W.KV_INT4, W.KV_F16])
@pytest.mark.parametrize("mode", [W.SCALE_NONE, W.SCALE_PER_TENSOR, W.SCALE_PER_CHANNEL])
def test_dequantize_all_codes_bit_exact(pa, kind, mode):
    rng = np.random.default_rng(3)
    if kind == W.KV_F16:
        codes = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.uint8)
        n = 65536
    elif kind == W.KV_INT4:
        codes = np.arange(256, dtype=np.uint8)  # every nibble pair
        n = 512
    else:
        codes = np.arange(256, dtype=np.uint8)
        n = 256
    ch = 64
    scale = np.exp(rng.uniform(-4, 4, ch)).astype(np.float32)
    say(f"dequantize kind={kind} mode={mode}")
    got = pa.pa_dequantize(kind, dev(codes), n, dev(scale) if mode else None, mode=mode,
                           channels=ch).cpu().numpy()
    ref = oracle.dequantize(kind, codes, n, scale, mode, ch)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    if kind == W.KV_E4M3:
        assert nan.sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def rtz_f16_of_bf16_bits(bits):
    """fp16 value of bf16 bits converted toward zero (numpy/torch arithmetic):
    the decode paged_attn_fwd applies to a BF16 cache."""
    x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = np.array(x)
    fin = np.isfinite(x)
    a = np.abs(x[fin])
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -24)))
    q = np.exp2(np.maximum(e, -14) - 10)  # fp16 spacing (subnormal below 2^-14)
    r = np.trunc(a / q) * q
    r = np.minimum(r, 65504.0)
    out[fin] = np.copysign(r, x[fin])
    return out


@pytest.mark.parametrize("mode", [W.SCALE_NONE, W.SCALE_PER_TENSOR, W.SCALE_PER_CHANNEL])
def test_dequantize_bf16_all_codes(pa, mode):
    """Every bf16 bit pattern: equal to the oracle's exact value wherever fp16
    holds it (magnitudes in [2^-14, 65504], zeros, infinities, NaN), and to the
    toward-zero fp16 value elsewhere."""
    rng = np.random.default_rng(4)
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n = 65536
    ch = 64
    scale = np.exp(rng.uniform(-4, 4, ch)).astype(np.float32)
    say(f"dequantize bf16 mode={mode}")
    got = pa.pa_dequantize(W.KV_BF16, dev(codes.view(np.uint8)), n,
                           dev(scale) if mode else None, mode=mode, channels=ch).cpu().numpy()
    ref = oracle.dequantize(W.KV_BF16, codes.view(np.uint8), n, scale, mode, ch)
    val = (codes.astype(np.uint32) << 16).view(np.float32)
    a = np.abs(val)
    exact = (a == 0) | ((a >= 2.0 ** -14) & (a <= 65504)) | np.isinf(val)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    m = exact & ~nan
    assert np.array_equal(got[m].view(np.uint32), ref[m].view(np.uint32))
    sc = np.ones(n, np.float32) if mode == 0 else (
        np.full(n, scale[0], np.float32) if mode == 1 else scale[np.arange(n) % ch])
    want = (rtz_f16_of_bf16_bits(codes).astype(np.float32) * sc)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _insert_gpu(pa, case):
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    if case.in_bf16:
        k = dev(case.k.view(np.int16)).view(torch.bfloat16)
        v = dev(case.v.view(np.int16)).view(torch.bfloat16)
    else:
        k, v = dev(case.k), dev(case.v)
    pa.kv_insert(kc, vc, k, v, dev(case.slot_mapping), kv_kind=case.kv_kind,
                 k_scale=None if case.k_scale is None else dev(case.k_scale),
                 v_scale=None if case.v_scale is None else dev(case.v_scale),
                 k_scale_mode=case.scale_mode, v_scale_mode=case.scale_mode)
    torch.cuda.synchronize()
    return kc.cpu().numpy(), vc.cpu().numpy()


def _insert_oracle(case):
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    oracle.kv_insert(kc, vc, case.kv_kind, case.k, case.v, case.slot_mapping,
                     k_scale=case.k_scale, k_scale_mode=case.scale_mode, v_scale=case.v_scale,
                     v_scale_mode=case.scale_mode, block_size=case.block_size,
                     in_is_bf16=case.in_bf16)
    return kc, vc


@pytest.mark.parametrize("kind,mode", [(W.KV_E4M3, W.SCALE_PER_TENSOR),
                                       (W.KV_INT8, W.SCALE_PER_CHANNEL),
                                       (W.KV_INT4, W.SCALE_PER_TENSOR),
                                       (W.KV_BF16, W.SCALE_NONE)])
def test_insert_bf16_input_bit_exact(pa, kind, mode):
    """bf16 input rows (and a BF16 cache), with slotless rows, slot -1 rows and
    rows whose slot lies past the cache: cache bytes equal the oracle's."""
    case = W.insert_case(31 + kind, T=600, Hkv=2, D=128, bs=16, kv_kind=kind, scale_mode=mode,
                         slotless_tail=5, neg_slots=3, value_scale=2.0, in_dtype="bf16",
                         oob_slots=4)
    say(f"insert bf16 kind={kind} mode={mode}")
    gk, gv = _insert_gpu(pa, case)
    ok, ov = _insert_oracle(case)
    assert np.array_equal(gk, ok) and np.array_equal(gv, ov)


def test_insert_slot_past_cache_skipped(pa):
    """A slot at or past num_blocks * block_size is not written (it would lie
    outside the cache); the other rows land exactly as the oracle's."""
    case = W.insert_case(77, T=300, Hkv=2, D=128, bs=16, kv_kind=W.KV_E4M3,
                         scale_mode=W.SCALE_PER_TENSOR, oob_slots=7)
    assert (case.slot_mapping >= case.num_blocks * case.block_size).sum() == 7
    say("insert slots past the cache")
    gk, gv = _insert_gpu(pa, case)
    ok, ov = _insert_oracle(case)
    assert np.array_equal(gk, ok) and np.array_equal(gv, ov)


@pytest.mark.parametrize("kind,mode", [(W.KV_E4M3, W.SCALE_PER_TENSOR),
                                       (W.KV_E4M3, W.SCALE_PER_CHANNEL),
                                       (W.KV_INT8, W.SCALE_PER_TENSOR),
                                       (W.KV_INT8, W.SCALE_PER_CHANNEL),
                                       (W.KV_INT4, W.SCALE_PER_TENSOR),
                                       (W.KV_INT4, W.SCALE_PER_CHANNEL),
                                       (W.KV_F16, W.SCALE_NONE)])
@pytest.mark.parametrize("T,tail", [(17, 0), (1024, 5), (2049, 5)])
def test_insert_bit_exact(pa, kind, mode, T, tail):
    """Token counts 17/1024/2049 with and without 5 slotless rows, plus rows with
    slot -1; destination prefilled with 0xFF; cache bytes compared exactly."""
    case = W.insert_case(T * 7 + kind, T=T + tail, Hkv=2, D=128, bs=16, kv_kind=kind,
                         scale_mode=mode, slotless_tail=tail, neg_slots=3, value_scale=2.0)
    say(f"insert kind={kind} mode={mode} T={T} tail={tail}")
    gk, gv = _insert_gpu(pa, case)
    ok, ov = _insert_oracle(case)
    assert np.array_equal(gk, ok) and np.array_equal(gv, ov)


def test_insert_e4m3_rounding_edges(pa):
    """Exact midpoints between E4M3 codes, subnormals, saturation: inserted
    codes equal the oracle's nearest-even, saturating encoder."""
    vals = oracle.e4m3_to_f32(np.arange(0x7E, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([mids, -mids, vals, [500.0, -700.0, 448.0, 1e-9, 0.0]])
    x = x[np.abs(x.astype(np.float16).astype(np.float64) - x) == 0]  # exactly fp16
    T = len(x) // 64
    x = x[:T * 64].astype(np.float16).reshape(T, 1, 64)
    case = W.InsertCase(k=x, v=x, slot_mapping=np.arange(T, dtype=np.int64) + 16, num_blocks=T // 16 + 3,
                        block_size=16, kv_kind=W.KV_E4M3, k_scale=np.ones(1, np.float32),
                        v_scale=np.ones(1, np.float32), scale_mode=W.SCALE_PER_TENSOR,
                        k_cache=np.full((T // 16 + 3, 16, 1, 64), 0xFF, np.uint8),
                        v_cache=np.full((T // 16 + 3, 16, 1, 64), 0xFF, np.uint8))
    say("insert e4m3 rounding edges")
    gk, _ = _insert_gpu(pa, case)
    ok, _ = _insert_oracle(case)
    assert np.array_equal(gk, ok)
