"""The indexer-to-attention chain -- kv_insert_mxfp4 -> paged_mqa_logits ->
pa_topk_select -> paged_attn_sparse, with a kv_insert into an E4M3 cache
beside it -- captured once in a HIP graph and replayed several times: every
replay reproduces the eager chain bit for bit (the inserted cache bytes of
both inserts, the logits, the ids and the attention output),
with eager runs of the chain between the replays. The eager chain's logits
and ids are also checked against the oracle's chain."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DevAttn, dev, say

pytestmark = pytest.mark.gpu


def chain_inputs():
    """One sequence of 700 tokens in blocks 1.. of an MXFP4 cache (block 64),
    two query rows, the E4M3 attention cache of the same sequence."""
    T, bs = 700, 64
    ins = W.mxfp4_insert_case(7101, T=T, in_dtype="f16", spread=3.0)
    ins.slot_mapping[:] = np.arange(bs, bs + T)
    cols = -(-T // 128) * 128 // bs
    bt = np.zeros((1, cols), np.int32)
    bt[0, :-(-T // bs)] = np.arange(1, 1 + -(-T // bs))
    assert bt.max() < ins.kv_fused.shape[0]
    lg = W.logits_case("graph_idx", 7102, B=1, next_n=2, H=64, D=128, bs=bs, lens=[T],
                       max_context_len=T)
    at = W.attn_case("graph_attn", 7103, B=1, next_n=2, Hq=16, Hkv=2, D=128, bs=32, lens=[T],
                     kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR, max_context_len=T)
    return ins, bt, lg, at


def test_chain_graph_replay_matches_eager(pa):
    ins, bt, lg, at = chain_inputs()
    T, k = 700, 256
    kv0 = dev(ins.kv_fused)
    kv = kv0.clone()
    keys = dev(ins.k_bits.view(np.int16)).view(torch.float16)
    slots = dev(ins.slot_mapping)
    q, sfq, w = dev(lg.q), dev(lg.sf_q), dev(lg.weights)
    lens, btd = dev(np.array([T], np.int32)), dev(bt)
    d = DevAttn(at)
    logits = torch.empty((2, T), dtype=torch.float32, device="cuda")
    sel = torch.empty((2, k), dtype=torch.int32, device="cuda")
    out = torch.empty(at.q.shape, dtype=torch.float16, device="cuda")
    lws_n = pa.paged_mqa_logits_workspace_size(q, sfq, kv, w, lens, btd, T)
    lws = torch.empty(max(lws_n, 1), dtype=torch.uint8, device="cuda")
    sws_n = pa.paged_attn_sparse_workspace_size(d.q, d.k, d.bt, T, at.kv_kind, k)
    sws = torch.empty(max(sws_n, 1), dtype=torch.uint8, device="cuda")
    fins = W.insert_case(7104, T=200, Hkv=2, D=128, bs=16, kv_kind=W.KV_E4M3,
                         scale_mode=W.SCALE_PER_TENSOR, value_scale=2.0)
    kc0, vc0 = dev(fins.k_cache), dev(fins.v_cache)
    kc, vc = kc0.clone(), vc0.clone()
    ik, iv, isl = dev(fins.k), dev(fins.v), dev(fins.slot_mapping)
    iks, ivs = dev(fins.k_scale), dev(fins.v_scale)

    def chain():
        pa.kv_insert(kc, vc, ik, iv, isl, kv_kind=fins.kv_kind, k_scale=iks, v_scale=ivs,
                     k_scale_mode=fins.scale_mode, v_scale_mode=fins.scale_mode)
        pa.kv_insert_mxfp4(kv, keys, slots)
        pa.paged_mqa_logits(q, sfq, kv, w, lens, btd, T, out=logits, workspace=lws)
        pa.topk_select(logits, lens, 2, k, sel=sel)
        pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, T, sel.view(1, 2, k),
                             kv_kind=at.kv_kind, k_scale=d.ks, v_scale=d.vs, workspace=sws)

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
        kv.copy_(kv0)
        logits.fill_(float("nan"))
        sel.fill_(-7)
        out.fill_(float("nan"))

    def snapshot():
        torch.cuda.synchronize()
        return (kv.cpu().numpy().copy(), logits.cpu().numpy().view(np.uint32).copy(),
                sel.cpu().numpy().copy(), out.cpu().numpy().view(np.uint16).copy(),
                kc.cpu().numpy().copy(), vc.cpu().numpy().copy())

    say("graph chain: eager")
    reset()
    chain()
    ref = snapshot()
    # the eager chain against the oracle's: insert, logits and ids bit for bit
    kv_o = oracle.mxfp4_insert(ins.kv_fused.copy(), ins.k_bits, ins.slot_mapping, in_dtype="f16")
    assert np.array_equal(ref[0], kv_o)
    lo = oracle.mqa_logits(lg.q, lg.sf_q, kv_o, lg.weights, np.array([T], np.int32), bt, T)
    assert np.array_equal(ref[1], lo.view(np.uint32))
    assert np.array_equal(ref[2], oracle.topk_select(lo, np.array([T], np.int32), 2, k))
    ok_, ov_ = fins.k_cache.copy(), fins.v_cache.copy()
    oracle.kv_insert(ok_, ov_, fins.kv_kind, fins.k, fins.v, fins.slot_mapping,
                     k_scale=fins.k_scale, k_scale_mode=fins.scale_mode, v_scale=fins.v_scale,
                     v_scale_mode=fins.scale_mode, block_size=fins.block_size)
    assert np.array_equal(ref[4], ok_) and np.array_equal(ref[5], ov_)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("graph chain: capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            chain()
    torch.cuda.current_stream().wait_stream(s)
    names = ("MXFP4 cache bytes", "logits", "ids", "attention output", "E4M3 K cache bytes",
             "E4M3 V cache bytes")
    for r in range(4):
        reset()
        torch.cuda.synchronize()
        say(f"graph chain: replay {r}")
        g.replay()
        got = snapshot()
        for name, a, b in zip(names, got, ref):
            assert np.array_equal(a, b), f"replay {r}: {name} differ from the eager chain"
        say(f"graph chain: eager run after replay {r}")
        reset()
        chain()
        got = snapshot()
        for name, a, b in zip(names, got, ref):
            assert np.array_equal(a, b), f"eager run {r}: {name} differ"
