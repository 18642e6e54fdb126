"""Pins for the oracle's selection-driven sparse paged attention and its
grouped union plan ("Stabilize QSA page4 order under KV relocation": selected
token ids per query row, a physical-page union with token masks, logical page
as the sort key; "Stop grouped-page4 null-block padding from leaking E4M3 NaN":
unselected and null tokens must not reach the output).

Independent references: the dense oracle (a selection of every token equals
non-causal dense attention), a numpy brute force over the selected tokens on
tiny inputs, set semantics of the selection (order, repeats, padding and
out-of-range ids change nothing), relocation invariance, NaN-poisoned tails
and null block, and numpy set arithmetic for the plan.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from tests import brute


def sparse_small(seed=1, kind=W.KV_E4M3, next_n=2, lens=(37, 70, 5), topk=24, bs=16):
    case = W.attn_case("sp", seed, B=len(lens), next_n=next_n, Hq=4, Hkv=2, D=64, bs=bs,
                       lens=list(lens), kv_kind=kind,
                       scale_mode=W.SCALE_NONE if kind == W.KV_F16 else W.SCALE_PER_TENSOR)
    return W.with_selection(case, seed + 100, topk, window=8)


def run(case, sel, lib):
    return oracle.paged_attn_sparse(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                    case.block_table, case.context_lens, sel, lib=lib,
                                    **case.oracle_kwargs())


def pin_full_selection_is_dense(lib):
    case, _ = sparse_small(2)
    L = case.context_lens
    sel = np.full((case.batch, case.next_n, int(L.max())), -1, np.int32)
    for b in range(case.batch):
        sel[b, :, :L[b]] = np.arange(L[b])
    dense = oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                              case.context_lens, lib=lib,
                              **{**case.oracle_kwargs(), "causal": False})
    assert np.array_equal(run(case, sel, lib), dense)


def pin_brute_force(lib):
    case, sel = sparse_small(3)
    got = run(case, sel, lib)
    K = brute.dequant_cache(case.k_cache, case.kv_kind, case.head_dim, case.k_scale,
                            case.k_scale_mode)
    V = brute.dequant_cache(case.v_cache, case.kv_kind, case.head_dim, case.v_scale,
                            case.v_scale_mode)
    G = case.num_q_heads // case.num_kv_heads
    q = case.q.astype(np.float64)
    for b in range(case.batch):
        L = int(case.context_lens[b])
        Kb = brute.gather(K, case.block_table[b], L, case.block_size)
        Vb = brute.gather(V, case.block_table[b], L, case.block_size)
        for i in range(case.next_n):
            S = sorted({int(t) for t in sel[b, i] if 0 <= t < L})
            for h in range(case.num_q_heads):
                if not S:
                    assert (got[b, i, h] == 0).all()
                    continue
                s = case.softmax_scale * (Kb[S, h // G] @ q[b, i, h])
                p = np.exp(s - s.max())
                ref = (p[:, None] * Vb[S, h // G]).sum(0) / p.sum()
                assert np.allclose(got[b, i, h], ref, rtol=1e-9, atol=1e-12)


def pin_selection_is_a_set(lib):
    case, sel = sparse_small(4)
    base = run(case, sel, lib)
    rng = np.random.default_rng(5)
    sel2 = sel.copy()
    for b in range(case.batch):
        for i in range(case.next_n):
            rng.shuffle(sel2[b, i])
    sel3 = np.concatenate([sel2, sel2[:, :, :3], np.full(sel.shape[:2] + (2,), 10 ** 6, np.int32)],
                          -1)
    assert np.array_equal(run(case, sel3, lib), base)


def pin_relocation_and_poison(lib):
    case, sel = sparse_small(6, kind=W.KV_E4M3)
    base = run(case, sel, lib)
    assert np.isfinite(base).all()  # NaN tails and block 0 are never selected
    moved = W.relocate(case, 7)
    assert np.array_equal(run(moved, sel, lib), base)


def pin_empty_rows(lib):
    case, sel = sparse_small(8)
    sel = sel.copy()
    sel[1, 0, :] = -1
    got = run(case, sel, lib)
    assert (got[1, 0] == 0).all() and np.abs(got[1, 1]).sum() > 0


def pin_plan(lib):
    case, sel = sparse_small(9, next_n=3, lens=(200, 64, 1, 0), topk=40, bs=16)
    entries, masks, count = oracle.sparse_plan(sel, case.block_table, case.context_lens, 16,
                                               lib=lib)
    for b in range(case.batch):
        L = int(case.context_lens[b])
        rows = [{int(t) for t in sel[b, i] if 0 <= t < L} for i in range(case.next_n)]
        pages = sorted({t // 16 for r in rows for t in r})
        n = int(count[b])
        assert n == len(pages)
        assert entries[b, :n, 1].tolist() == pages  # ascending logical order
        assert entries[b, :n, 0].tolist() == [int(case.block_table[b, p]) for p in pages]
        for e, p in enumerate(pages):
            for i in range(case.next_n):
                want = sum(1 << (t - 16 * p) for t in rows[i] if t // 16 == p)
                assert int(masks[b, e, i]) == want


ALL_PINS = [pin_full_selection_is_dense, pin_brute_force, pin_selection_is_a_set,
            pin_relocation_and_poison, pin_empty_rows, pin_plan]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_sparse_pin(orc, pin):
    pin(orc)
