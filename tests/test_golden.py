"""Values the pages print, kept as cited fixtures under tests/golden/, checked
against the oracle's codecs and arithmetic and against the library's host-side
contract checks (CPU only: no GPU call is made)."""
import ctypes
import os

import numpy as np

import oracle
import paged_attention_quantized_amd as pa
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fixture(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        k, v = (s.strip() for s in line.split("=", 1))
        vals[k] = v.split()
    return vals


def test_fold_overflow_example(orc):
    g = fixture("fold_overflow.txt")
    q, ks = float(g["q"][0]), float(g["k_scale"][0])
    with np.errstate(over="ignore", invalid="ignore"):
        f16 = np.float16(q) * np.float16(ks)
        assert np.isinf(f16) and g["fold_fp16"] == ["inf"]
        assert np.isnan(f16 * np.float16(0.0)) and g["fold_fp16_times_zero"] == ["nan"]
    assert np.float32(q) * np.float32(ks) == np.float32(g["fold_fp32"][0])
    # the oracle computes that case through the normalized route: finite, and the
    # mean of V when every score is 0 (the closed form of the worked case)
    case = W.attn_case("golden_fold", 31, B=1, next_n=1, Hq=2, Hkv=1, D=64, bs=16, lens=[5],
                       kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                       v_scale_range=(0.5, 2.0))
    case.q[:] = np.float16(q)
    case.k_scale = np.full((1, 64), ks, np.float32)
    case.k_cache[:] = 0
    out = oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                            case.context_lens, **case.oracle_kwargs())
    assert np.isfinite(out).all()
    vdeq = oracle.dequantize(W.KV_INT8, case.v_cache[case.block_table[0, 0], :5, 0].reshape(-1),
                             5 * 64, case.v_scale.reshape(-1), W.SCALE_PER_CHANNEL, 64)
    mean = vdeq.reshape(5, 64).astype(np.float64).mean(0)
    assert np.allclose(out[0, 0, 0], mean, rtol=1e-6, atol=1e-6)
    ratio = int(g["int8_scale_divisor"][0]) / int(g["int4_scale_divisor"][0])
    assert round(ratio) == int(g["int4_over_int8_ratio_approx"][0])


def test_null_block_values(orc):
    g = fixture("null_block.txt")
    nan_codes = [int(c, 16) for c in g["e4m3_nan_codes"]]
    dec = oracle.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    assert sorted(np.flatnonzero(np.isnan(dec)).tolist()) == sorted(nan_codes)
    bits = oracle.f64_to_f16(np.array([dec[nan_codes[0]]], np.float64))
    assert int(np.asarray(bits).view(np.uint16)[0]) == int(g["e4m3_nan_as_fp16_bits"][0], 16)
    assert (int(g["microblock_tokens"][0]) * int(g["microblock_dims"][0])
            == int(g["microblock_value_bytes"][0]))
    # 480 NaN outputs = every row and head of the tile on each poisoned dim
    assert (int(g["tile_rows"][0]) * int(g["tile_heads"][0]) * len(g["poisoned_dims"])
            == int(g["nan_count_unfixed_decode_like"][0]))
    assert float(g["agreement_bound_after_fix"][0]) < 2e-3  # inside the output tolerance


def test_fp4_api_values():
    g = fixture("fp4_api.txt")
    D, sf = int(g["head_dim"][0]), int(g["sf_vec_size"][0])
    assert D // 2 + D // sf == int(g["kv_row_bytes"][0])
    case = W.logits_case("golden_rows", 5, B=1, next_n=1, H=16, D=D, bs=64, lens=[70],
                         max_context_len=128)
    assert case.kv_fused.shape[-1] == int(g["kv_row_bytes"][0])
    spi, bs = int(g["sf_interleave_sf_per_int32"][0]), int(g["sf_interleave_block_size"][0])
    slots = [(k % spi) * (bs // spi) + k // spi for k in range(8)]
    assert slots == [int(x) for x in g["sf_interleave_slot_to_token"]]


def test_fp4_block_table_rule_is_enforced():
    """The host check of paged_mqa_logits rejects a table one column short of
    round_up(len, 128) / block_size and accepts the printed column count (the
    call then fails only on its null data pointers; nothing reaches a GPU)."""
    g = fixture("fp4_api.txt")
    L, bs, cols = (int(g[k][0]) for k in ("table_rule_context_len", "table_rule_block_size",
                                          "table_rule_columns"))
    lib = pa.load()

    def status(ncols):
        a = pa.LogitsArgs(out=None, out_row_stride=L, q=None, sf_q=None, kv_fused=None,
                          weights=None, context_lens=None, block_table=None, batch=1, next_n=1,
                          num_heads=64, head_dim=128, block_size=bs, max_blocks_per_seq=ncols,
                          num_blocks=16, max_context_len=L, sf_vec_size=32)
        return lib.paged_mqa_logits(ctypes.byref(a), None, 0, None)

    assert status(cols - 1) == 3  # PA_ERR_PRECONDITION
    assert status(cols) == 1      # PA_ERR_INVALID_ARG: the null pointers, past the rule


def test_relocation_diff_is_one_fp16_ulp():
    g = fixture("relocation.txt")
    d = float(g["max_abs_diff_before_fix"][0])
    assert d == 2.0 ** -11 == float(np.spacing(np.float16(0.5)))
    assert int(g["differing_elements_after_fix"][0]) == 0
