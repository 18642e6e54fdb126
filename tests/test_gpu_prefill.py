"""GPU parity of paged_attn_fwd with more than 32 query rows per KV head
(long verify and chunked prefill: the rows run in blocks of 32, each block
walking only the tokens its last row can see) against the oracle, through the
C ABI.

Tolerance as for the other attention tests: |gpu - oracle| <= max(2e-3,
1 fp16 ulp of the oracle value). Rows are independent, so at full size the
first and last query steps of a sequence are checked against the oracle run
on just those steps: the last k steps over the same length, the first k over
length L - next_n + k (the causal rule puts row i at L - next_n + i).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import (DevAttn, compare_attn, compare_attn_conditioned, log_parity,
                            oracle_attn, run_attn, say)

pytestmark = pytest.mark.gpu


def prefill_cases():
    """Row counts that leave ragged last blocks, blocks that split the heads of
    one step, rows that see nothing, both KV-scale modes, every kind."""
    return [
        W.attn_case("pf_e4m3_n64_g4", 3101, B=3, next_n=64, Hq=8, Hkv=2, D=128, bs=16,
                    lens=[300, 64, 40], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR),
        W.attn_case("pf_int8_perchan_n16_g8", 3102, B=2, next_n=16, Hq=16, Hkv=2, D=256, bs=32,
                    lens=[700, 20], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                    q_dist=(-100.0, 100.0), zero_k_channel_frac=0.1,
                    v_scale_range=(1e-2, 65504.0 / 127)),
        W.attn_case("pf_f16_n33_g1", 3103, B=2, next_n=33, Hq=2, Hkv=2, D=64, bs=16,
                    lens=[100, 33], kv_kind=W.KV_F16, scale_mode=W.SCALE_NONE),
        W.attn_case("pf_e4m3_g48_n1", 3104, B=3, next_n=1, Hq=48, Hkv=1, D=128, bs=32,
                    lens=[513, 7, 1], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR),
        W.attn_case("pf_e4m3_g12_n3", 3105, B=2, next_n=3, Hq=24, Hkv=2, D=128, bs=16,
                    lens=[77, 2], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR),
        W.attn_case("pf_int4_n20_g4", 3106, B=2, next_n=20, Hq=8, Hkv=2, D=128, bs=32,
                    lens=[260, 19], kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_TENSOR),
        W.attn_case("pf_e4m3_noncausal_n40", 3107, B=2, next_n=40, Hq=4, Hkv=2, D=64, bs=16,
                    lens=[90, 45], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR,
                    causal=False),
        # 128 rows or more per KV head: the prefill layout (256-row groups, one
        # head per workgroup, stages decoded once into LDS)
        W.attn_case("pg_int8_perchan_n32_g8", 3108, B=2, next_n=32, Hq=16, Hkv=2, D=128, bs=32,
                    lens=[700, 20], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                    q_dist=(-100.0, 100.0), zero_k_channel_frac=0.1,
                    v_scale_range=(1e-2, 65504.0 / 127)),
        W.attn_case("pg_int4_n40_g4", 3109, B=3, next_n=40, Hq=8, Hkv=2, D=128, bs=32,
                    lens=[260, 19, 45], kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_TENSOR),
        W.attn_case("pg_f16_d64_n75_g4", 3110, B=2, next_n=75, Hq=8, Hkv=2, D=64, bs=16,
                    lens=[500, 80], kv_kind=W.KV_F16, scale_mode=W.SCALE_NONE),
        W.attn_case("pg_e4m3_d64_noncausal_n64", 3111, B=2, next_n=64, Hq=4, Hkv=2, D=64, bs=16,
                    lens=[90, 130], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR,
                    causal=False),
        W.attn_case("pg_e4m3_n128_g1", 3112, B=3, next_n=128, Hq=4, Hkv=4, D=128, bs=32,
                    lens=[1000, 128, 3], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR),
        # one step's 64 heads span two waves; 5 steps = 320 rows = 2 groups
        W.attn_case("pg_e4m3_g64_n5", 3113, B=2, next_n=5, Hq=64, Hkv=1, D=128, bs=16,
                    lens=[333, 4], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR),
        # INT8 per-channel at head_dim 64, 3 groups with a ragged last one
        W.attn_case("pg_int8_perchan_d64_n100_g6", 3114, B=2, next_n=100, Hq=12, Hkv=2, D=64,
                    bs=32, lens=[400, 150], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                    q_dist=(-100.0, 100.0), zero_k_channel_frac=0.1,
                    v_scale_range=(1e-2, 65504.0 / 127)),
    ]


@pytest.mark.parametrize("idx", range(14))
def test_prefill_small_parity(pa, idx):
    case = prefill_cases()[idx]
    say(f"prefill parity {case.name} B={case.batch} next_n={case.next_n} "
        f"lens={list(case.context_lens)}")
    got = run_attn(pa, case)
    ref = oracle_attn(case)
    r = compare_attn(got, ref, case.name)
    say(f"{case.name}: max err/tol = {r:.3f}")
    if case.causal:
        for b in range(case.batch):
            L = int(case.context_lens[b])
            for i in range(case.next_n):
                if L - case.next_n + i < 0:  # sees no token: +0
                    assert np.all(got[b, i].view(np.uint16) == 0)


@pytest.mark.parametrize("idx", [0, 1, 7, 9])
def test_prefill_relocation_bit_identical(pa, idx):
    case = prefill_cases()[idx]
    say(f"prefill relocation {case.name}")
    base = run_attn(pa, case)
    for other in (W.relocate(case, 31), W.unpaged(case)):
        got = run_attn(pa, other)
        assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


def last_steps(case, k):
    return dataclasses.replace(case, q=np.ascontiguousarray(case.q[:, -k:]))


def first_steps(case, k):
    L = np.maximum(case.context_lens.astype(np.int64) - case.next_n + k, 0).astype(np.int32)
    return dataclasses.replace(case, q=np.ascontiguousarray(case.q[:, :k]), context_lens=L)


def test_step_slices_match_full_oracle():
    """The slicing used at full size, checked against the full oracle on a
    small case (host only, but next to the test that relies on it)."""
    case = prefill_cases()[0]
    full = oracle_attn(case)
    assert np.array_equal(oracle_attn(last_steps(case, 5)), full[:, -5:])
    assert np.array_equal(oracle_attn(first_steps(case, 7)), full[:, :7])


def test_full_fp8_prefill(pa):
    """The benchmark's workload in its launch configuration: every query row
    of every sequence against the oracle, and a relocation of all pages
    bit-identical."""
    case = W.fp8_prefill()
    say(f"full {case.name}: B={case.batch} next_n={case.next_n} "
        f"tokens={int(case.context_lens.sum())}")
    got = run_attn(pa, case)
    assert not np.isnan(got.astype(np.float32)).any()
    say("full prefill: oracle")
    ref, cond, vr = oracle_attn(case, conditioning=True)
    st = compare_attn_conditioned(got, ref, cond, vr, case.name)
    say(f"{case.name}: {st}")
    log_parity({"test": "full", "case": case.name, **st})
    other = run_attn(pa, W.relocate(case, 41))
    assert np.array_equal(other.view(np.uint16), got.view(np.uint16))
