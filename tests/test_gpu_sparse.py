"""GPU parity of paged_attn_sparse (the selection-driven QSA route of
"Stabilize QSA page4 order under KV relocation", with the zero rule for
unattended rows of "Stop grouped-page4 null-block padding from leaking E4M3
NaN") against the oracle, through the C ABI.

Tolerance: as for paged_attn_fwd, |gpu - oracle| <= max(2e-3, 1 fp16 ulp of
the oracle value) per element. Bitwise: the union plan equals the oracle's,
the output is identical under physical relocation and under any reordering,
repetition or padding of the selection, rows that select nothing are +0, and
no NaN comes out of NaN-poisoned null blocks and tails.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import (DevAttn, compare_attn, compare_attn_conditioned, dev, log_parity,
                            say)

pytestmark = pytest.mark.gpu


def small_cases():
    """(case, sel) pairs the oracle finishes in seconds: both kinds, RT 1 and 2,
    head dims 64 / 128 / 256, block sizes 16 and 32, ragged and empty sequences."""
    out = []
    c = W.attn_case("sp_e4m3_d128", 2101, B=5, next_n=2, Hq=8, Hkv=2, D=128, bs=16,
                    lens=[300, 37, 1, 0, 129], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    out.append(W.with_selection(c, 2201, 48, window=16))
    c = W.attn_case("sp_f16_d64_rt2", 2102, B=3, next_n=4, Hq=16, Hkv=2, D=64, bs=32,
                    lens=[500, 70, 33], kv_kind=W.KV_F16, scale_mode=W.SCALE_NONE)
    out.append(W.with_selection(c, 2202, 64, window=8))
    c = W.attn_case("sp_e4m3_d256", 2103, B=3, next_n=1, Hq=16, Hkv=4, D=256, bs=32,
                    lens=[1000, 65, 7], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    out.append(W.with_selection(c, 2203, 100, window=32))
    c = W.attn_case("sp_e4m3_verify", 2104, B=3, next_n=4, Hq=64, Hkv=8, D=128, bs=32,
                    lens=[900, 40, 5], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    out.append(W.with_selection(c, 2204, 96, window=24))
    c = W.attn_case("sp_f16_nosel_scale", 2105, B=2, next_n=3, Hq=4, Hkv=4, D=128, bs=16,
                    lens=[64, 200], kv_kind=W.KV_F16, scale_mode=W.SCALE_NONE)
    out.append(W.with_selection(c, 2205, 5, window=2))
    # integer kinds with per-channel K and V scales (the fold of the dense path)
    c = W.attn_case("sp_int8_perchan", 2106, B=3, next_n=2, Hq=16, Hkv=2, D=256, bs=32,
                    lens=[800, 97, 3], kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_CHANNEL,
                    q_dist=(-100.0, 100.0), zero_k_channel_frac=0.1,
                    v_scale_range=(1e-2, 65504.0 / 127))
    out.append(W.with_selection(c, 2206, 80, window=20))
    c = W.attn_case("sp_int4_perchan", 2108, B=2, next_n=4, Hq=8, Hkv=1, D=128, bs=16,
                    lens=[600, 45], kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_CHANNEL,
                    q_dist=(-100.0, 100.0), zero_k_channel_frac=0.1)
    out.append(W.with_selection(c, 2208, 70, window=10))
    c = W.attn_case("sp_int4_pt_rt2", 2109, B=2, next_n=4, Hq=32, Hkv=4, D=256, bs=32,
                    lens=[333, 64], kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_TENSOR)
    out.append(W.with_selection(c, 2209, 50, window=12))
    return out


def run_sparse(pa, case, sel, workspace=None):
    d = DevAttn(case)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, dev(sel),
                         kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                         k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
                         softmax_scale=case.softmax_scale, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_sparse(case, sel):
    return oracle.paged_attn_sparse(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                    case.block_table, case.context_lens, sel,
                                    **case.oracle_kwargs())


def empty_rows(case, sel):
    B, N = sel.shape[:2]
    e = np.zeros((B, N), bool)
    for b in range(B):
        L = int(case.context_lens[b])
        for i in range(N):
            e[b, i] = not ((sel[b, i] >= 0) & (sel[b, i] < L)).any()
    return e


@pytest.mark.parametrize("idx", range(8))
def test_sparse_small_parity(pa, idx):
    case, sel = small_cases()[idx]
    say(f"sparse parity {case.name} B={case.batch} next_n={case.next_n} "
        f"lens={list(case.context_lens)} topk={sel.shape[2]}")
    got = run_sparse(pa, case, sel)
    ref, cond, vr = oracle.paged_attn_sparse(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                             case.block_table, case.context_lens, sel,
                                             conditioning=True, **case.oracle_kwargs())
    st = compare_attn_conditioned(got, ref, cond, vr, case.name)
    e = empty_rows(case, sel)
    assert np.all(got[e].view(np.uint16) == 0)  # +0 bits
    say(f"{case.name}: {st}, empty rows {int(e.sum())}")


def test_sparse_plan_probe(pa):
    """The planner's union, logical order and masks equal the oracle's plan."""
    for case, sel in small_cases():
        d = DevAttn(case)
        say(f"sparse plan {case.name}")
        cap = case.block_table.shape[1]
        entries, masks, count = pa.pa_sparse_plan(
            dev(sel), d.bt, d.cl, case.max_context_len, q_shape=case.q.shape,
            k_cache_shape=case.k_cache.shape, kv_kind=case.kv_kind,
            k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode, cap=cap)
        torch.cuda.synchronize()
        e, m, n = entries.cpu().numpy(), masks.cpu().numpy().view(np.uint32), count.cpu().numpy()
        re, rm, rn = oracle.sparse_plan(sel, case.block_table, case.context_lens,
                                        case.block_size, cap=cap)
        assert np.array_equal(n, rn)
        for b in range(case.batch):
            assert np.array_equal(e[b, :n[b]], re[b, :rn[b]])
        assert np.array_equal(m, rm)


@pytest.mark.parametrize("idx", [0, 3, 5, 6])
def test_sparse_relocation_and_selection_order_bit_identical(pa, idx):
    case, sel = small_cases()[idx]
    say(f"sparse relocation {case.name}")
    base = run_sparse(pa, case, sel)
    for seed in (5, 6):
        got = run_sparse(pa, W.relocate(case, seed), sel)
        assert np.array_equal(got.view(np.uint16), base.view(np.uint16))
    rng = np.random.default_rng(9)
    sel2 = sel.copy()
    for b in range(case.batch):
        for i in range(case.next_n):
            rng.shuffle(sel2[b, i])
    sel3 = np.ascontiguousarray(np.concatenate(
        [sel2, sel2[:, :, :5], np.full(sel.shape[:2] + (3,), -7, np.int32)], -1))
    got = run_sparse(pa, case, sel3)
    assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


def test_sparse_full_selection_matches_dense_oracle(pa):
    """Selecting every token of every row is non-causal dense attention."""
    case = W.attn_case("sp_full", 2106, B=3, next_n=2, Hq=8, Hkv=2, D=128, bs=16,
                       lens=[130, 16, 1], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR,
                       causal=False)
    L = case.context_lens
    sel = np.full((case.batch, case.next_n, int(L.max())), -1, np.int32)
    for b in range(case.batch):
        sel[b, :, :L[b]] = np.arange(L[b])
    say("sparse full selection")
    got = run_sparse(pa, case, sel)
    ref = oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                            case.context_lens, **case.oracle_kwargs())
    compare_attn(got, ref, case.name)


def test_sparse_empty_selection_and_dirty_workspace(pa):
    """topk 0 and all-invalid selections write +0 everywhere; a workspace full
    of garbage from an earlier call changes nothing."""
    case, sel = small_cases()[0]
    say("sparse empty selection")
    none = np.full(sel.shape[:2] + (0,), -1, np.int32)
    got = run_sparse(pa, case, none)
    assert np.all(got.view(np.uint16) == 0)
    bad = np.full(sel.shape, -1, np.int32)
    bad[:, :, 0] = 10 ** 6
    got = run_sparse(pa, case, bad)
    assert np.all(got.view(np.uint16) == 0)
    base = run_sparse(pa, case, sel)
    d = DevAttn(case)
    need = pa.paged_attn_sparse_workspace_size(d.q, d.k, d.bt, case.max_context_len,
                                               case.kv_kind, sel.shape[2], case.k_scale_mode,
                                               case.v_scale_mode)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    got = run_sparse(pa, case, sel, workspace=ws)
    assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


def test_sparse_args_errors(pa):
    case, sel = small_cases()[0]
    d = DevAttn(case)
    out = torch.empty(case.q.shape, dtype=torch.float16, device="cuda")
    # more than 4 query steps per sequence: no sparse kernel
    i8 = W.attn_case("sp_i8", 2107, B=1, next_n=5, Hq=4, Hkv=1, D=128, bs=16, lens=[20],
                     kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_TENSOR)
    di = DevAttn(i8)
    with pytest.raises(pa.PaError, match="UNSUPPORTED"):
        pa.paged_attn_sparse(torch.empty(i8.q.shape, dtype=torch.float16, device="cuda"), di.q,
                             di.k, di.v, di.bt, di.cl, i8.max_context_len,
                             dev(np.zeros((1, 5, 4), np.int32)), kv_kind=i8.kv_kind,
                             k_scale=di.ks, v_scale=di.vs)
    with pytest.raises(pa.PaError, match="WORKSPACE"):
        pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, dev(sel),
                             kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                             workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))


def test_full_fp8_sparse_verify(pa):
    """The benchmark's workload in its launch configuration; every sequence
    against the oracle, then a relocation of all pages (bit-identical)."""
    case, sel = W.fp8_sparse_verify()
    say(f"full {case.name}: B={case.batch} tokens={int(case.context_lens.sum())} "
        f"topk={sel.shape[2]}")
    got = run_sparse(pa, case, sel)
    assert not np.isnan(got.astype(np.float32)).any()
    ref, cond, vr = oracle.paged_attn_sparse(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                             case.block_table, case.context_lens, sel,
                                             conditioning=True, **case.oracle_kwargs())
    st = compare_attn_conditioned(got, ref, cond, vr, case.name)
    say(f"{case.name}: {st}")
    log_parity({"test": "full", "case": case.name, **st})
    other = run_sparse(pa, W.relocate(case, 21), sel)
    assert np.array_equal(other.view(np.uint16), got.view(np.uint16))


def clustered_selection(case, seed):
    """Selections made of spans, as a clustered top-k gives them: a head span
    every row selects (whole 16-token sub-tiles), a span only some rows select,
    and for each row its own recent tokens; pages whose second half nobody
    selects and sub-tiles every row selects in full both occur."""
    rng = np.random.default_rng(seed)
    B, N = case.batch, case.next_n
    rows = []
    for b in range(B):
        L = int(case.context_lens[b])
        per = []
        for i in range(N):
            ids = set(range(min(L, 48)))                       # shared head: 3 full sub-tiles
            if L > 200 and i % 2 == 0:
                ids |= set(range(128, 144))                    # half a 32-token page, some rows
            a = int(rng.integers(0, max(1, L - 20)))
            ids |= set(range(a, min(L, a + int(rng.integers(1, 20)))))  # a short private span
            ids |= set(range(max(0, L - 8 - i), L))            # the row's own recent tokens
            per.append(sorted(ids))
        rows.append(per)
    topk = max(len(r) for per in rows for r in per)
    sel = np.full((B, N, topk), -1, np.int32)
    for b in range(B):
        for i in range(N):
            r = np.array(rows[b][i], np.int32)
            rng.shuffle(r)
            sel[b, i, :r.size] = r
    return sel


@pytest.mark.parametrize("kind,bs", [(W.KV_E4M3, 32), (W.KV_F16, 16), (W.KV_E4M3, 16)])
def test_sparse_clustered_selection(pa, kind, bs):
    """Sub-tiles no row selected are skipped and sub-tiles every row selected
    run unmasked: the result still equals the oracle, and a relocation of the
    pages leaves it bit-identical."""
    case = W.attn_case(f"sp_cluster_{kind}_{bs}", 2301 + bs, B=3, next_n=4, Hq=16, Hkv=2,
                       D=128, bs=bs, lens=[600, 260, 30], kv_kind=kind,
                       scale_mode=W.SCALE_NONE if kind == W.KV_F16 else W.SCALE_PER_TENSOR)
    sel = clustered_selection(case, 2400 + bs)
    say(f"sparse clustered {case.name} topk={sel.shape[2]}")
    got = run_sparse(pa, case, sel)
    compare_attn(got, oracle_sparse(case, sel), case.name)
    moved = run_sparse(pa, W.relocate(case, 77), sel)
    assert np.array_equal(moved.view(np.uint16), got.view(np.uint16))
