"""Planted mistakes: each mutation below is a plausible slip in the oracle (a
dropped term, a wrong sign, index, bias or rounding rule, a transposed
operand). The test copies oracle.c, applies one mutation, builds the copy on
the CPU and runs the pins against it; at least one pin must fail. This shows
the pins constrain every part of the oracle rather than restating it.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from tests import (test_oracle_attn, test_oracle_insert, test_oracle_logits, test_oracle_mxfp4,
                   test_oracle_sparse, test_oracle_topk)


def pin_codec_e4m3(lib):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f32(codes, lib)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    vals = ref[:0x7E].astype(np.float64)
    x = np.concatenate([((vals[:-1] + vals[1:]) / 2), np.linspace(-460, 460, 3001)]).astype(
        np.float32)
    enc = oracle.f32_to_e4m3(x, lib)
    want = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(enc, want.numpy())


def pin_codec_round(lib):
    y = [2.5, 3.5, -2.5, 0.5, 1.5, 126.5, 200.0, -9.0]
    for lim in (127, 7):
        assert [lib.orc_round_clamp(v, lim) for v in y] == \
            np.clip(np.rint(np.float32(y)), -lim, lim).astype(int).tolist()


PINS = ([pin_codec_e4m3, pin_codec_round] + test_oracle_attn.ALL_PINS +
        test_oracle_logits.ALL_PINS + test_oracle_insert.ALL_PINS + test_oracle_mxfp4.ALL_PINS +
        test_oracle_sparse.ALL_PINS + test_oracle_topk.ALL_PINS)

MUTATIONS = {
    "gqa_head_map": ("for (int h = hk * group; h < (hk + 1) * group; ++h) {\n        int64_t row",
                     "for (int h = hk; h < Hq; h += Hkv) {\n        int64_t row", 0),
    "causal_off_by_one": ("if (causal && pos + 1 < nvis) nvis = pos + 1;",
                          "if (causal && pos < nvis) nvis = pos;"),
    "softmax_sign": ("s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);", 0),
    "dropped_normalizer": ("for (int d = 0; d < D; ++d) orow[d] /= l;", "", 0),
    "dropped_softmax_scale": ("s[t] = (double)softmax_scale * acc;", "s[t] = acc;", 0),
    # reads the [Hkv, D] scale as [D, Hkv]; every per-channel pin uses Hkv = 2, so it stays
    # in bounds
    "per_channel_transposed": ("if (mode == ORC_SCALE_PER_CHANNEL) return scale[hk * D + d];",
                               "if (mode == ORC_SCALE_PER_CHANNEL) return scale[d * 2 + hk];"),
    "e4m3_bias": ("v = ldexpf(8.0f + (float)m, e - 10);", "v = ldexpf(8.0f + (float)m, e - 9);"),
    "e4m3_ties_up": ("- a);\n    if (d < bestd || (d == bestd && (c & 1) == 0)) {",
                     "- a);\n    if (d < bestd || (d == bestd)) {"),
    "int4_nibble_order": ("int nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);\n    return",
                          "int nib = (d % 2 == 0) ? (byte >> 4) : (byte & 15);\n    return"),
    "v_slot_index": ("deq(v_cache, kind, v_scale, v_mode, blk, t % bs, hk,",
                     "deq(v_cache, kind, v_scale, v_mode, blk, (t + 1) % bs, hk,"),
    "f16_exponent": ("v = ldexp(1024.0 + f, e - 25);", "v = ldexp(1024.0 + f, e - 24);"),
    "int_round_away": ("float r = nearbyintf(y);", "float r = roundf(y);"),
    "logits_weight_row": ("acc = epi_step(weights[r * H + h], sh, acc, epi_format);",
                          "acc = epi_step(weights[h], sh, acc, epi_format);"),
    "logits_epi_unrounded_sum": ("return epi_round(fmaf(epi_round(w, epi_format), "
                                 "epi_round(s, epi_format), acc), epi_format);",
                                 "return fmaf(epi_round(w, epi_format), "
                                 "epi_round(s, epi_format), acc);"),
    "logits_epi_f16_as_bf16": ("if (epi_format == 1) return orc_f16_to_f32(orc_f64_to_f16(",
                               "if (epi_format == 1) return orc_bf16_to_f32(orc_f32_to_bf16(("
                               "float)"),
    "logits_sf_offset": ("const uint8_t* ksf = base + (int64_t)bs * (D / 2) +\n",
                         "const uint8_t* ksf = base +\n"),
    "logits_sf_interleave_swapped": ("if ((k % spi) * (bs / spi) + k / spi == t) return k;",
                                     "if ((k / spi) * (bs / spi) + k % spi == t) return k;"),
    "logits_relu_inverted": ("if (relu) sh = sh > 0.0f ? sh : 0.0f;",
                             "if (relu) sh = sh < 0.0f ? sh : 0.0f;"),
    "logits_tail_zero": ("orow[t] = -INFINITY;", "orow[t] = 0.0f;"),
    "logits_q_scale_byte": ("((qsf >> (8 * g)) & 0xFF)", "((qsf >> (8 * (3 - g))) & 0xFF)"),
    "insert_offset": ("int off = (int)(slot % bs);", "int off = (int)(slot % bs) ^ 1;"),
    "insert_bf16_input_as_f16": ("return in_is_bf16 ? orc_bf16_to_f32(x[idx]) : orc_f16_to_f32(x[idx]);",
                                 "return orc_f16_to_f32(x[idx]);"),
    "mx_scale_offset": ("int b = (e - 1) - 2 + 127;", "int b = (e - 1) - 1 + 127;"),
    "e2m1_ties_odd": ("float d = fabsf(a - orc_e2m1_to_f32((uint8_t)c));\n"
                      "    if (d < bestd || (d == bestd && (c & 1) == 0)) {",
                      "float d = fabsf(a - orc_e2m1_to_f32((uint8_t)c));\n"
                      "    if (d < bestd || (d == bestd && (c & 1) == 1)) {"),
    "mx_nibble_order": ("data[d / 2] = (uint8_t)((data[d / 2] & 0xF0) | c);",
                        "data[d / 2] = (uint8_t)((data[d / 2] & 0x0F) | (c << 4));"),
    "sparse_range_unchecked": ("if (sel_row[j] >= 0 && sel_row[j] < L) mark[sel_row[j]] = 1;",
                               "if (sel_row[j] >= 0 && sel_row[j] < L - 1) mark[sel_row[j]] = 1;"),
    "sparse_plan_mask_bit": ("rowmask[i] |= 1u << j;", "rowmask[i] |= 1u << (j ^ 1);"),
    "sparse_row_selection": ("mark + (size_t)i * n, L, D, softmax_scale,",
                             "mark, L, D, softmax_scale,"),
    "cond_gap_uses_first": ("if (s[t] > second) second = s[t];",
                            "if (s[t] > second && second == -INFINITY) second = s[t];"),
    "cond_eps_drops_length": ("(D + 8) * ldexp(1.0, -24) * aabs", "8 * ldexp(1.0, -24) * aabs"),
    "cond_range_misses_ties": ("if (!vis[t] || s[t] < m - 8.0 * eps - 32.0) continue;",
                               "if (!vis[t] || s[t] < m) continue;"),
    "cond_sens_signed": ("vsens[d] += s[t] * fabs((double)vd[(int64_t)t * D + d] - orow[d]);",
                         "vsens[d] += s[t] * ((double)vd[(int64_t)t * D + d] - orow[d]);"),
    "topk_ties_to_higher_id": ("return (a->t > b->t) - (a->t < b->t);",
                               "return (a->t < b->t) - (a->t > b->t);"),
    "topk_nan_first": ("if (an != bn) return an ? 1 : -1;", "if (an != bn) return an ? -1 : 1;"),
    "topk_tail_candidates": ("for (int t = 0; t < L; ++t) {\n      c[t].v = logit_value(",
                             "for (int t = 0; t < L; ++t) {\n      c[t].v = t + 1 == L ? 1e30f : logit_value("),
    "mx_sf_token_order": ("(int64_t)sf_slot_of_token(pos, bs, spi, sf_interleaved) * spi;",
                          "(int64_t)pos * spi;"),
}


def test_unmutated_passes_all_pins(orc):
    for pin in PINS:
        pin(orc)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new, *which = MUTATIONS[name]
    if which:  # the anchor recurs (dense and sparse attention): mutate occurrence which[0]
        at = -1
        for _ in range(which[0] + 1):
            at = src.index(old, at + 1)
        mutated = src[:at] + new + src[at + len(old):]
    else:
        assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
        mutated = src.replace(old, new)
    path = tmp_path / "oracle_mut.c"
    path.write_text(mutated)
    so = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", *oracle.CFLAGS, str(path), "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    failures = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lib)
        except (AssertionError, ValueError):  # ValueError: the oracle rejected its input
            failures.append(pin.__name__)
            break
    assert failures, f"no pin caught the planted mistake {name}"
