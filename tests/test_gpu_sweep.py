"""Seeded random sweep of paged_attn_fwd and paged_attn_sparse shapes against
the oracle, through the C ABI, plus HIP-graph replays of the sparse and the
prefill paths.

Each case draws the KV kind and scale mode, head_dim, block size, KV heads,
query heads per KV head, query steps (up to prefill-sized row counts, so the
ring kernel's dense, row-block and the prefill layouts are all exercised),
the causal flag, fp16 or bf16 queries and ragged lengths including empty
sequences. Values span the input generator's full ranges: per-tensor INT
scales uniform in [0.01, 2], per-channel K and V scales log-uniform in
[1e-2, 1e3] (INT8 V up to 65504/127) with q uniform in [-100, 100] and 10% of
K channels zero. Tolerance: |gpu - oracle| <= max(2e-3, 1 ulp of the output
type at the oracle value); rows whose fp64 top-2 score gap is below 8x the
fp32 score-error bound are classified ill-conditioned and checked for lying
within the V range of the tokens that can carry weight (the counts are
printed and, with $PA_PARITY_LOG set, logged). Rows that see no token are +0.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import (DevAttn, compare_attn, compare_attn_conditioned, dev, log_parity,
                            oracle_attn, run_attn, say, to_f64)

pytestmark = pytest.mark.gpu

N_DENSE = 72
N_SPARSE = 12


def dense_case(i):
    rng = np.random.default_rng(5000 + i)
    kind = [W.KV_F16, W.KV_E4M3, W.KV_INT8, W.KV_INT4][i % 4]
    D = int(rng.choice([128, 256] if kind == W.KV_INT4 else [64, 128, 256]))
    bs = int(rng.choice([16, 32]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 12, 16]))
    # mostly decode / verify, every third case prefill-sized
    next_n = int(rng.integers(24, 80)) if i % 3 == 2 else int(rng.integers(1, 6))
    while next_n * G * D > 48 * 1024:  # keep the oracle to seconds
        next_n = max(1, next_n // 2)
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 600, B)]
    if i % 5 == 0:
        lens[0] = 0
    if kind == W.KV_F16:
        mode = W.SCALE_NONE
    elif kind == W.KV_E4M3:
        mode = W.SCALE_PER_TENSOR
    else:
        mode = [W.SCALE_PER_TENSOR, W.SCALE_PER_CHANNEL][i % 2]
    kw = {}
    if mode == W.SCALE_PER_CHANNEL:
        # the generator's per-channel distribution: K and V scales log-uniform in
        # [1e-2, 1e3] (INT8 V up to 65504/127 so V stays finite in fp16), q in
        # [-100, 100], 10% of K channels zero
        kw = dict(zero_k_channel_frac=0.1, q_dist=(-100.0, 100.0),
                  v_scale_range=(1e-2, 65504.0 / 127) if kind == W.KV_INT8 else (1e-2, 1e3))
    return W.attn_case(f"sweep{i}_k{kind}_d{D}_bs{bs}_h{Hkv}x{G}_n{next_n}", 6000 + i, B=B,
                       next_n=next_n, Hq=Hkv * G, Hkv=Hkv, D=D, bs=bs, lens=lens, kv_kind=kind,
                       scale_mode=mode, causal=bool(i % 4 != 3),
                       max_context_len=max(1, max(lens)), **kw)


def bf16_query(i):
    return i % 5 == 1


@pytest.mark.parametrize("i", range(N_DENSE))
def test_dense_sweep(pa, i):
    case = dense_case(i)
    bf = bf16_query(i)
    say(f"sweep {case.name} lens={list(case.context_lens)} causal={case.causal} bf16={bf}")
    d = DevAttn(case, bf16=bf)
    got = to_f64(d.run(pa))
    ref, cond, vr = oracle_attn(case, conditioning=True, q=d.q.cpu() if bf else None)
    st = compare_attn_conditioned(got, ref, cond, vr, case.name, "bf16" if bf else "f16")
    say(f"{case.name}: {st}")
    log_parity({"test": "dense_sweep", "case": case.name, "bf16": bf, **st})


def sparse_case(i):
    rng = np.random.default_rng(7000 + i)
    kind = [W.KV_F16, W.KV_E4M3, W.KV_INT8, W.KV_INT4][i % 4]
    D = int(rng.choice([128, 256] if kind == W.KV_INT4 else [64, 128, 256]))
    bs = int(rng.choice([16, 32]))
    Hkv = int(rng.choice([1, 2, 4]))
    next_n = int(rng.integers(1, 5))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if g * next_n <= 32]))
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 900, B)]
    if kind == W.KV_F16:
        mode = W.SCALE_NONE
    elif kind == W.KV_E4M3:
        mode = W.SCALE_PER_TENSOR
    else:
        mode = [W.SCALE_PER_TENSOR, W.SCALE_PER_CHANNEL][(i // 4) % 2]
    kw = {}
    if mode == W.SCALE_PER_CHANNEL:
        kw = dict(zero_k_channel_frac=0.1, q_dist=(-100.0, 100.0),
                  v_scale_range=(1e-2, 65504.0 / 127) if kind == W.KV_INT8 else (1e-2, 1e3))
    case = W.attn_case(f"ssweep{i}_k{kind}_s{mode}_d{D}_bs{bs}_h{Hkv}x{G}_n{next_n}", 8000 + i,
                       B=B, next_n=next_n, Hq=Hkv * G, Hkv=Hkv, D=D, bs=bs, lens=lens,
                       kv_kind=kind, scale_mode=mode, max_context_len=max(1, max(lens)), **kw)
    return W.with_selection(case, 9000 + i, int(rng.integers(1, 120)),
                            window=int(rng.integers(1, 40)))


def run_sparse(pa, case, sel, workspace=None, out=None, bf16=False):
    d = DevAttn(case, bf16=bf16)
    if out is None:
        out = torch.full(case.q.shape, float("nan"), dtype=d.q.dtype, device="cuda")
    pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, dev(sel),
                         kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                         k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
                         softmax_scale=case.softmax_scale, workspace=workspace)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("i", range(N_SPARSE))
def test_sparse_sweep(pa, i):
    case, sel = sparse_case(i)
    bf = bf16_query(i)
    say(f"sparse sweep {case.name} lens={list(case.context_lens)} topk={sel.shape[2]} bf16={bf}")
    out = run_sparse(pa, case, sel, bf16=bf)
    got = to_f64(out)
    q = DevAttn(case, bf16=True).q.cpu() if bf else case.q
    ref, cond, vr = oracle.paged_attn_sparse(q, case.k_cache, case.v_cache, case.kv_kind,
                                             case.block_table, case.context_lens, sel,
                                             conditioning=True, **case.oracle_kwargs())
    st = compare_attn_conditioned(got, ref, cond, vr, case.name, "bf16" if bf else "f16")
    say(f"{case.name}: {st}")
    log_parity({"test": "sparse_sweep", "case": case.name, "bf16": bf, **st})


def replay_check(eager, out, g, again):
    """Replay the captured graph several times, with an eager call on the same
    workspace between replays; every replay and every eager call equal the
    first eager output bitwise."""
    for k in range(4):
        out.fill_(float("nan"))
        say(f"graph replay {k}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.view(np.uint16)), k
        assert np.array_equal(again().view(np.uint16), eager.view(np.uint16))


def test_sparse_graph_replay(pa):
    case, sel = sparse_case(3)
    d = DevAttn(case)
    sl = dev(sel)
    n = pa.paged_attn_sparse_workspace_size(d.q, d.k, d.bt, case.max_context_len, case.kv_kind,
                                            sel.shape[2], case.k_scale_mode, case.v_scale_mode)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("sparse graph replay: eager reference")
    again = lambda: run_sparse(pa, case, sel, workspace=ws).cpu().numpy()
    eager = again()
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, sl,
                                 kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                                 k_scale_mode=case.k_scale_mode,
                                 v_scale_mode=case.v_scale_mode,
                                 softmax_scale=case.softmax_scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    replay_check(eager, out, g, again)


def test_prefill_graph_replay(pa):
    case = W.attn_case("pf_graph", 8100, B=2, next_n=40, Hq=16, Hkv=2, D=128, bs=32,
                       lens=[500, 60], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    assert case.next_n * case.num_q_heads // case.num_kv_heads >= 128  # the prefill layout
    d = DevAttn(case)
    n = pa.paged_attn_workspace_size(d.q, d.k, d.bt, case.max_context_len, case.kv_kind,
                                     case.k_scale_mode, case.v_scale_mode)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("prefill graph replay: eager reference")
    again = lambda: d.run(pa, workspace=ws).cpu().numpy()
    eager = again()
    compare_attn(eager, oracle_attn(case), case.name)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.paged_attn_fwd(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len,
                              kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                              k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
                              softmax_scale=case.softmax_scale, causal=case.causal,
                              workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    replay_check(eager, out, g, again)
