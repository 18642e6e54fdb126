"""Pins for the oracle's paged attention.

What fixes the values, independently of oracle.c:
  * fp64 brute force: torch scaled_dot_product_attention on K/V gathered through
    the block table and decoded by library casts (tests/brute.py);
  * invariance under relocation of physical pages and equality with an unpaged
    (contiguous) layout, bit for bit;
  * the worked case of "Normalize the PER_CHANNEL K scale folded into Q for paged
    XQA" (Description and Validation status): q = 100, k_scale = 1000 and every
    K code zero must give a finite result; every score is then 0 and the
    closed form is the mean of the visible V rows;
  * L = 1 gives the single dequantized V row exactly;
  * poisoned null block (page 0 as the null block, "Stop grouped-page4
    null-block padding from leaking E4M3 NaN", Root cause) and poisoned tail
    slots do not change the result.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests import brute


def tiny_cases():
    """Small inputs covering every KV kind, scale mode, GQA, causal next_n > 1,
    ragged tails, a page-multiple length, and an empty sequence."""
    cases = []
    cases.append(W.tiny_f16())
    cases.append(W.attn_case("e4m3_pt", 5, B=3, next_n=1, Hq=4, Hkv=2, D=32, bs=8,
                             lens=[13, 16, 1], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR))
    cases.append(W.attn_case("int8_pc_causal", 6, B=2, next_n=3, Hq=6, Hkv=2, D=16, bs=4,
                             lens=[9, 4], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                             q_dist=(-2.0, 2.0), k_scale_range=(1e-2, 1e-1),
                             v_scale_range=(0.1, 2.0), zero_k_channel_frac=0.25))
    cases.append(W.attn_case("int4_pc", 7, B=2, next_n=2, Hq=4, Hkv=2, D=32, bs=8,
                             lens=[21, 0], kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_CHANNEL,
                             q_dist=(-1.0, 1.0), k_scale_range=(1e-2, 1e-1),
                             v_scale_range=(0.1, 2.0), causal=False, max_context_len=21))
    cases.append(W.attn_case("int8_pt_nocausal", 8, B=2, next_n=2, Hq=2, Hkv=1, D=16, bs=4,
                             lens=[7, 12], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_TENSOR,
                             causal=False))
    cases.append(W.attn_case("bf16", 9, B=1, next_n=1, Hq=2, Hkv=2, D=16, bs=4, lens=[10],
                             kv_kind=W.KV_BF16, scale_mode=W.SCALE_NONE))
    return cases


def run_oracle(case, lib):
    return oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                             case.context_lens, lib=lib, **case.oracle_kwargs())


# --- pins as functions of a loaded oracle library, so the planted-mistake test
# --- can run them against mutated builds


def pin_brute_force(lib):
    for case in tiny_cases():
        got = run_oracle(case, lib)
        ref = brute.attention_sdpa(case)
        scale = max(1.0, float(np.abs(ref).max()))
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * scale, err_msg=case.name)


def pin_relocation_and_unpaged(lib):
    for case in tiny_cases():
        base = run_oracle(case, lib)
        for other in (W.relocate(case, 99), W.unpaged(case)):
            got = run_oracle(other, lib)
            assert np.array_equal(got.view(np.uint64), base.view(np.uint64)), case.name


def worked_case(kind, qval, kscale, seed=21):
    case = W.attn_case("worked", seed, B=2, next_n=1, Hq=4, Hkv=2, D=32, bs=8, lens=[19, 40],
                       kv_kind=kind, scale_mode=W.SCALE_PER_TENSOR if kind == W.KV_E4M3
                       else W.SCALE_PER_CHANNEL, v_scale_range=(0.5, 2.0))
    case.q[:] = np.float16(qval)
    case.k_scale = np.full((2, 32), kscale, np.float32)
    case.k_scale_mode = W.SCALE_PER_CHANNEL
    if case.v_scale is not None and case.v_scale.size == 1:
        case.v_scale = np.full((2, 32), case.v_scale[0], np.float32)
        case.v_scale_mode = W.SCALE_PER_CHANNEL
    case.k_cache[:] = 0  # every K code zero (E4M3 0x00 is +0)
    return case


def pin_worked_case(lib):
    for kind in (W.KV_INT4, W.KV_INT8, W.KV_E4M3):
        for qval, kscale in ((100.0, 1000.0), (100.0, 1e4)):  # q*k_scale = 1e5 and 1e6
            case = worked_case(kind, qval, kscale)
            got = run_oracle(case, lib)
            assert np.isfinite(got).all()
            V = brute.dequant_cache(case.v_cache, kind, 32, case.v_scale, case.v_scale_mode)
            for b in range(case.batch):
                L = int(case.context_lens[b])
                mean = brute.gather(V, case.block_table[b], L, 8).astype(np.float64).mean(0)
                for h in range(4):
                    np.testing.assert_allclose(got[b, 0, h], mean[h // 2], rtol=1e-12,
                                               atol=1e-12)


def pin_single_token(lib):
    for kind, mode in ((W.KV_E4M3, W.SCALE_PER_TENSOR), (W.KV_INT4, W.SCALE_PER_CHANNEL),
                       (W.KV_F16, W.SCALE_NONE)):
        case = W.attn_case("one", 31, B=2, next_n=1, Hq=4, Hkv=2, D=16, bs=4, lens=[1, 1],
                           kv_kind=kind, scale_mode=mode, q_dist=(-3.0, 3.0),
                           k_scale_range=(0.1, 1.0), v_scale_range=(0.1, 1.0))
        got = run_oracle(case, lib)
        V = brute.dequant_cache(case.v_cache, kind, 16, case.v_scale, case.v_scale_mode)
        for b in range(2):
            v0 = V[case.block_table[b, 0], 0].astype(np.float64)  # [Hkv, D]
            for h in range(4):
                assert np.array_equal(got[b, 0, h], v0[h // 2])


def pin_poison_insensitive(lib):
    for case in tiny_cases():
        base = run_oracle(case, lib)
        rng = np.random.default_rng(1)
        k2, v2 = case.k_cache.copy(), case.v_cache.copy()
        k2[0] = rng.integers(0, 256, k2[0].shape, dtype=np.uint8)
        v2[0] = rng.integers(0, 256, v2[0].shape, dtype=np.uint8)
        bs = case.block_size
        for b in range(case.batch):
            L = int(case.context_lens[b])
            if L % bs:
                last = case.block_table[b, L // bs]
                k2[last, L % bs:] = 0x11
                v2[last, L % bs:] = 0x22
        other = W.AttnCase(**{**case.__dict__, "k_cache": k2, "v_cache": v2})
        got = run_oracle(other, lib)
        assert np.array_equal(got.view(np.uint64), base.view(np.uint64)), case.name


def pin_bf16_q(lib):
    """bf16 queries: the oracle reads their bits as bf16 (brute force on the
    same values through torch's bfloat16 cast)."""
    import dataclasses

    import torch
    for case in tiny_cases()[1:4]:
        qb = torch.from_numpy(case.q.astype(np.float32) * 3.0).to(torch.bfloat16)
        got = oracle.paged_attn(qb, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                                case.context_lens, lib=lib, **case.oracle_kwargs())
        ref = brute.attention_sdpa(dataclasses.replace(case, q=qb.float().numpy()))
        scale = max(1.0, float(np.abs(ref).max()))
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * scale, err_msg=case.name)


def pin_thread_count_invariant(lib):
    """The parallel loops split independent units: 1 or 5 threads give the
    same bits."""
    case = tiny_cases()[2]
    oracle.set_threads(1, lib)
    one = run_oracle(case, lib)
    oracle.set_threads(5, lib)
    five = run_oracle(case, lib)
    oracle.set_threads(0, lib)
    assert np.array_equal(one.view(np.uint64), five.view(np.uint64))


def brute_conditioning(case):
    """fp64 scores from library-decoded K, their top-2 gap, the fp32
    score-error bound (the formula stated in orc_paged_attn's header) and the
    V range over the relevant tokens, per output row."""
    D = case.head_dim
    K = brute.dequant_cache(case.k_cache, case.kv_kind, D, case.k_scale, case.k_scale_mode)
    C = brute.decode_cache(case.k_cache, case.kv_kind, D)
    V = brute.dequant_cache(case.v_cache, case.kv_kind, D, case.v_scale, case.v_scale_mode)
    fold = case.k_scale_mode == W.SCALE_PER_CHANNEL
    kmax = float(np.abs(case.k_scale).max()) if fold else 0.0
    B, N, Hq, _ = case.q.shape
    G = Hq // case.num_kv_heads
    out = {}
    for b in range(B):
        L = int(case.context_lens[b])
        kb = brute.gather(K, case.block_table[b], L, case.block_size).astype(np.float64)
        cb = brute.gather(C, case.block_table[b], L, case.block_size).astype(np.float64)
        vb = brute.gather(V, case.block_table[b], L, case.block_size).astype(np.float64)
        for i in range(N):
            nvis = min(L, L - N + i + 1) if case.causal else L
            for h in range(Hq):
                hk = h // G
                if nvis <= 0:
                    continue
                q = case.q[b, i, h].astype(np.float64)
                prod = q[None, :] * kb[:nvis, hk]
                s = case.softmax_scale * prod.sum(1)
                eps = case.softmax_scale * ((D + 8) * 2.0 ** -24 * np.abs(prod).sum(1) +
                                            2.0 ** -25 * kmax * np.abs(cb[:nvis, hk]).sum(1))
                srt = np.sort(s)
                gap = srt[-1] - srt[-2] if nvis >= 2 else np.inf
                e = eps.max()
                rel = s >= srt[-1] - 8 * e - 32
                p = np.exp(s - srt[-1])
                o = (p[:, None] * vb[:nvis, hk]).sum(0) / p.sum()
                sens = (p[:, None] * np.abs(vb[:nvis, hk] - o[None, :])).sum(0) / p.sum()
                out[(b, i, h)] = (gap, e, rel.sum(), vb[:nvis, hk][rel].min(0),
                                  vb[:nvis, hk][rel].max(0), sens)
    return out


def pin_conditioning(lib):
    """The conditioning outputs: gap, bound and sensitivity to rounding, the
    relevant-set size and V range exactly; a planted exact tie gives gap 0."""
    cases = tiny_cases()[1:5]
    tie = W.attn_case("tie", 41, B=1, next_n=1, Hq=2, Hkv=1, D=16, bs=4, lens=[9],
                      kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_TENSOR)
    tie.k_cache[tie.block_table[0, 1], 1] = tie.k_cache[tie.block_table[0, 0], 2]  # K_5 = K_2
    tie.q[0, 0, 0] = 0
    tie.q[0, 0, 0, 0] = np.float16(1.0)
    tie.k_cache[:, :, :, 0] = 0
    tie.k_cache[tie.block_table[0, 0], 2, 0, 0] = 100
    tie.k_cache[tie.block_table[0, 1], 1, 0, 0] = 100  # tokens 2 and 5 tie at the top
    for case in cases + [tie]:
        _, cond, vr = oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                        case.block_table, case.context_lens, lib=lib,
                                        conditioning=True, **case.oracle_kwargs())
        for (b, i, h), (gap, e, n, lo, hi, sens) in brute_conditioning(case).items():
            c = cond[b, i, h]
            if np.isinf(gap):
                assert np.isinf(c[0])
            else:
                np.testing.assert_allclose(c[0], gap, rtol=1e-9, atol=1e-9 * (1 + abs(e)))
            np.testing.assert_allclose(c[1], e, rtol=1e-9)
            assert c[2] == n, (case.name, b, i, h)
            assert np.array_equal(vr[b, i, h, 0], lo) and np.array_equal(vr[b, i, h, 1], hi)
            np.testing.assert_allclose(vr[b, i, h, 2], sens, rtol=1e-9,
                                       atol=1e-12 * (1 + np.abs(hi).max()))
    _, cond, _ = oracle.paged_attn(tie.q, tie.k_cache, tie.v_cache, tie.kv_kind, tie.block_table,
                                   tie.context_lens, lib=lib, conditioning=True,
                                   **tie.oracle_kwargs())
    assert cond[0, 0, 0, 0] == 0.0


ALL_PINS = [pin_brute_force, pin_relocation_and_unpaged, pin_worked_case, pin_single_token,
            pin_poison_insensitive, pin_bf16_q, pin_thread_count_invariant, pin_conditioning]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_attention_pin(orc, pin):
    pin(orc)


def test_unnormalized_fp16_fold_is_the_hazard():
    """Negative control for the worked case: storing q*k_scale in fp16 overflows
    (100 * 1000 > 65504) and a zero code then turns inf into NaN."""
    folded = np.float16(100.0) * np.float16(1000.0)
    assert np.isinf(folded)
    with np.errstate(invalid="ignore"):
        assert np.isnan(folded * np.float16(0.0))
    # the normalized fold is bounded by max|q|
    ks = np.array([1e-2, 3.0, 1000.0], np.float32)
    assert np.all(np.abs(np.float16(100.0) * (ks / ks.max())) <= 100.0)


def test_multiplicative_mask_leaks_nan():
    """Negative control for null-block padding: a probability of exactly 0 times
    an E4M3 NaN value is NaN, which is why padded rows must be zeroed or never
    read ("Stop grouped-page4 null-block padding ...", Root cause)."""
    p = np.array([0.0, 1.0])
    v = np.array([np.nan, 2.0])
    with np.errstate(invalid="ignore"):
        assert np.isnan(p @ v)
    assert (p @ np.where(p > 0, v, 0.0)) == 2.0


def test_oracle_rejects_visible_null_block(orc):
    case = W.tiny_f16()
    bt = case.block_table.copy()
    bt[0, 1] = 0  # a visible token now maps to the null block
    bad = W.AttnCase(**{**case.__dict__, "block_table": bt})
    with pytest.raises(ValueError):
        run_oracle(bad, orc)
