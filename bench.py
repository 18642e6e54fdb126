"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the workload's entry point over its whole batch, inputs
resident in HBM: paged_attn_fwd (attention kernel and split merge),
paged_attn_sparse (union planner, attention, merge), paged_mqa_logits,
pa_topk_select over the logits, or kv_insert_mxfp4. The default workload is
FP8 E4M3 paged decode (batch 64, 32 query / 8 KV heads, head_dim 128,
block 16, context lengths uniform in [512, 4096], seed 1001). KV pools are
replicated and rotated so consecutive steps do not hit the 256 MB Infinity
Cache. Prints one JSON line: the wall-clock step rate, the dominant kernel's
own time (events on its dispatch), the same steps replayed from a HIP graph,
the device's streaming-read ceiling, and the oracle timed on the host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak

WORKLOADS = ("fp8_decode", "int8_perchan", "int4_perchan", "fp8_verify", "fp8_sparse_verify",
             "fp8_prefill", "mxfp4_logits", "mxfp4_topk", "mxfp4_insert")
METRIC = "FP8-KV paged decode: effective KV GB/s and % of MI355X HBM peak; tokens/s"


class Hip:
    """hipEvent helpers through ctypes (events on the stream the kernels run on)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


# ---------------------------------------------------------------------------
# algorithmic work of one call
# ---------------------------------------------------------------------------

def attn_bytes(case):
    """Algorithmic bytes of one call: K+V codes of visible tokens, the block-table
    entries of visible pages and the scales (q and out are counted apart)."""
    import workloads as W

    L = case.context_lens.astype("int64")
    kv = int(L.sum()) * case.num_kv_heads * W.row_bytes(case.kv_kind, case.head_dim) * 2
    pages = int(((L + case.block_size - 1) // case.block_size).sum())
    scales = sum(0 if s is None else s.nbytes for s in (case.k_scale, case.v_scale))
    return kv + 4 * pages + scales, case.q.nbytes * 2


def attn_flops(case):
    """Matrix flops of one call: 2 D for q.k and 2 D for p.v per (query row,
    head, visible token), the visible tokens of row i being those t <= L - next_n + i
    under the causal rule (all L otherwise)."""
    import numpy as np

    L = case.context_lens.astype(np.int64)[:, None]
    i = np.arange(case.next_n, dtype=np.int64)[None, :]
    vis = np.clip(L - case.next_n + i + 1, 0, L) if case.causal else \
        np.broadcast_to(L, (len(L), case.next_n))
    return int(vis.sum()) * case.num_q_heads * 4 * case.head_dim


def sparse_bytes(case, sel):
    """Algorithmic bytes of one sparse call: K+V codes of every page in the union
    of the rows' selections (whole pages are read) and the plan entries and
    masks the attention kernel reads (q, out and the selection apart)."""
    import numpy as np

    import workloads as W

    bs = case.block_size
    pages = 0
    for b in range(case.batch):
        L = int(case.context_lens[b])
        t = sel[b].ravel()
        pages += np.unique(t[(t >= 0) & (t < L)] // bs).size
    per_page = bs * case.num_kv_heads * W.row_bytes(case.kv_kind, case.head_dim) * 2
    scales = sum(0 if s is None else s.nbytes for s in (case.k_scale, case.v_scale))
    return pages * per_page + pages * (8 + 4 * case.next_n) + scales, pages


def logits_bytes(case):
    """KV bytes of visible tokens (FP4 data and scale bytes), the table entries
    of visible blocks and the fp32 output rows (max_context_len columns)."""
    L = case.context_lens.astype("int64")
    D = case.head_dim
    kv = int(L.sum()) * (D // 2 + D // 32)
    pages = int(((L + case.block_size - 1) // case.block_size).sum())
    out = case.batch * case.next_n * case.max_context_len * 4
    return kv + 4 * pages + out


def topk_bytes(case):
    """Logits read (visible tokens of every row, fp32) and ids written."""
    L = case.context_lens.astype("int64")
    return int(L.sum()) * case.next_n * 4 + case.batch * case.next_n * TOPK * 4


TOPK = 2048  # tokens selected per query row (the sparse workload's selection size)


# ---------------------------------------------------------------------------
# workloads: device setup, prepared calls, oracle sample
# ---------------------------------------------------------------------------

def npools_for(args, pool_bytes):
    return 1 if args.no_rotate else max(1, math.ceil((1 << 30) / pool_bytes))


class Bench:
    """One workload: `calls(stream)` gives one prepared call per KV pool on that
    stream; `oracle_sample(n)` runs the oracle on the first n units (sequences,
    or rows for the insert) and returns the fraction of one call's work done."""

    def __init__(self, name):
        self.name = name


def setup_attn(args, torch, pa, case, name):
    import numpy as np

    b = Bench(name)
    b.alg_bytes, b.other_bytes = attn_bytes(case)
    rows = case.next_n * case.num_q_heads // case.num_kv_heads
    prefill = rows >= 128 and case.head_dim <= 128
    b.tag = ("attn_prefill_" if prefill else "attn_ring_") + name
    b.npools = npools_for(args, case.k_cache.nbytes + case.v_cache.nbytes)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(b.npools - 1)]
    q, bt, cl = dev(case.q), dev(case.block_table), dev(case.context_lens)
    ks = None if case.k_scale is None else dev(case.k_scale)
    vs = None if case.v_scale is None else dev(case.v_scale)
    out = torch.empty(case.q.shape, dtype=torch.float16, device="cuda")
    ws_n = pa.paged_attn_workspace_size(q, kc, bt, case.max_context_len, case.kv_kind,
                                        case.k_scale_mode, case.v_scale_mode)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    b.calls = lambda s: [pa.prepare_paged_attn_fwd(
        out, q, kk, vv, bt, cl, case.max_context_len, kv_kind=case.kv_kind, k_scale=ks,
        v_scale=vs, k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
        softmax_scale=case.softmax_scale, causal=case.causal, workspace=ws, stream=s)
        for kk, vv in pools]
    b.extra = {"query_tokens": case.batch * case.next_n,
               "kv_tokens": int(case.context_lens.astype("int64").sum())}
    b.config = {"workload": name, "batch": case.batch, "next_n": case.next_n,
                "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                "head_dim": case.head_dim, "block_size": case.block_size,
                "max_context_len": case.max_context_len,
                "kv_dtype": {0: "f16", 1: "bf16", 2: "e4m3", 3: "int8", 4: "int4"}[case.kv_kind],
                "scales": {0: "none", 1: "per_tensor", 2: "per_channel"}[case.k_scale_mode],
                "causal": bool(case.causal)}
    if rows > 32:
        b.config["query_rows_per_kv_head"] = rows
    b.dtype = "f16xf16->f32"
    b.flops = attn_flops(case) if prefill else None
    full_flops = attn_flops(case)

    def oracle_sample(n):
        import oracle

        sub = case.sub_batch(list(range(n)))
        if prefill:
            # the last 16 query steps of each sampled sequence (the oracle's
            # cost is per query row): a causal chunk's last rows see the most
            m = min(16, case.next_n)
            import dataclasses
            sub = dataclasses.replace(sub, q=np.ascontiguousarray(sub.q[:, -m:]))
        oracle.paged_attn(sub.q, sub.k_cache, sub.v_cache, sub.kv_kind, sub.block_table,
                          sub.context_lens, **sub.oracle_kwargs())
        return attn_flops(sub) / full_flops
    b.oracle_sample = oracle_sample
    b.units = case.batch
    b.unit_name = "sequences" + (" (their last 16 query steps)" if prefill else "")
    return b


def setup_sparse(args, torch, pa, case_sel, name):
    import numpy as np

    case, sel = case_sel
    b = Bench(name)
    b.alg_bytes, pages = sparse_bytes(case, sel)
    b.other_bytes = case.q.nbytes * 2 + sel.nbytes
    b.tag = "attn_ring_" + name
    b.npools = npools_for(args, case.k_cache.nbytes + case.v_cache.nbytes)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(b.npools - 1)]
    q, bt, cl, sl = dev(case.q), dev(case.block_table), dev(case.context_lens), dev(sel)
    ks = None if case.k_scale is None else dev(case.k_scale)
    vs = None if case.v_scale is None else dev(case.v_scale)
    out = torch.empty(case.q.shape, dtype=torch.float16, device="cuda")
    ws_n = pa.paged_attn_sparse_workspace_size(q, kc, bt, case.max_context_len, case.kv_kind,
                                               sel.shape[2], case.k_scale_mode,
                                               case.v_scale_mode)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    b.calls = lambda s: [pa.prepare_paged_attn_sparse(
        out, q, kk, vv, bt, cl, case.max_context_len, sl, kv_kind=case.kv_kind, k_scale=ks,
        v_scale=vs, k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
        softmax_scale=case.softmax_scale, workspace=ws, stream=s) for kk, vv in pools]
    selected = 0
    for bb in range(case.batch):
        L = int(case.context_lens[bb])
        for i in range(case.next_n):
            t = sel[bb, i]
            selected += np.unique(t[(t >= 0) & (t < L)]).size
    b.extra = {"query_tokens": case.batch * case.next_n, "kv_tokens": int(selected),
               "union_pages": int(pages)}
    b.config = {"workload": name, "batch": case.batch, "next_n": case.next_n,
                "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                "head_dim": case.head_dim, "block_size": case.block_size,
                "max_context_len": case.max_context_len, "kv_dtype": "e4m3",
                "scales": "per_tensor", "topk": int(sel.shape[2]) - 4,
                "selection": "last 512 tokens + uniform earlier ones per row, seed 1006",
                "union_pages": int(pages)}
    b.dtype = "f16xf16->f32"
    b.flops = None

    def oracle_sample(n):
        import oracle

        sub = case.sub_batch(list(range(n)))
        ss = np.ascontiguousarray(sel[:n])
        oracle.paged_attn_sparse(sub.q, sub.k_cache, sub.v_cache, sub.kv_kind, sub.block_table,
                                 sub.context_lens, ss, **sub.oracle_kwargs())
        return sparse_bytes(sub, ss)[0] / b.alg_bytes
    b.oracle_sample = oracle_sample
    b.units = case.batch
    b.unit_name = "sequences"
    return b


def logits_sub(case, n):
    import dataclasses

    N = case.next_n
    return dataclasses.replace(case, q=case.q[:n], sf_q=case.sf_q[:n],
                               weights=case.weights[:n * N], context_lens=case.context_lens[:n],
                               block_table=case.block_table[:n])


def setup_logits(args, torch, pa, case, name, topk=False):
    import numpy as np

    b = Bench(name)
    b.npools = npools_for(args, case.kv_fused.nbytes)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = dev(case.kv_fused)
    pools = [kv] + [kv.clone() for _ in range(b.npools - 1)]
    q, sfq, w = dev(case.q), dev(case.sf_q), dev(case.weights)
    cl, bt = dev(case.context_lens), dev(case.block_table)
    out = torch.empty((case.batch * case.next_n, case.max_context_len), dtype=torch.float32,
                      device="cuda")
    b.extra = {"query_tokens": case.batch * case.next_n,
               "kv_tokens": int(case.context_lens.astype("int64").sum())}
    b.config = {"workload": name, "batch": case.batch, "next_n": case.next_n,
                "heads": case.num_heads, "head_dim": case.head_dim,
                "block_size": case.block_size, "max_context_len": case.max_context_len,
                "context_lens": "uniform [1, 32768], seed 1004", "kv_dtype": "mxfp4"}
    b.flops = None
    b.units = case.batch
    b.unit_name = "sequences"
    if topk:
        # the logits are computed once; a step selects the top 2048 of every row
        pa.paged_mqa_logits(q, sfq, pools[0], w, cl, bt, case.max_context_len, out=out)
        torch.cuda.synchronize()
        sel = torch.empty((case.batch * case.next_n, TOPK), dtype=torch.int32, device="cuda")
        b.npools = 1
        b.alg_bytes = topk_bytes(case)
        b.other_bytes = 0
        b.tag = "topk_" + name
        b.calls = lambda s: [pa.prepare_topk_select(out, cl, case.next_n, TOPK, sel=sel,
                                                    stream=s)]
        b.config["topk"] = TOPK
        b.dtype = "f32 keys->int32 ids"
        host_logits = out.cpu().numpy()

        def oracle_sample(n):
            import oracle

            oracle.topk_select(host_logits[:n * case.next_n], case.context_lens[:n],
                               case.next_n, TOPK)
            return topk_bytes(logits_sub(case, n)) / b.alg_bytes
    else:
        b.alg_bytes = logits_bytes(case)
        b.other_bytes = case.q.nbytes + case.sf_q.nbytes + case.weights.nbytes
        b.tag = "logits_" + name
        b.calls = lambda s: [pa.prepare_paged_mqa_logits(
            q, sfq, kvp, w, cl, bt, case.max_context_len, out=out, stream=s) for kvp in pools]
        b.dtype = "fp4xfp4->f32"

        def oracle_sample(n):
            import oracle

            sub = logits_sub(case, n)
            oracle.mqa_logits(sub.q, sub.sf_q, sub.kv_fused, sub.weights, sub.context_lens,
                              sub.block_table, sub.max_context_len)
            return logits_bytes(sub) / b.alg_bytes
    b.oracle_sample = oracle_sample
    return b


def setup_mxfp4_insert(args, torch, pa, case, name):
    import numpy as np

    b = Bench(name)
    T, D = case.k_bits.shape
    per_row = 2 * D + D // 2 + D // 32 + 8
    b.alg_bytes, b.other_bytes = T * per_row, 0
    b.tag = "mxfp4_insert"
    b.npools = 1
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = dev(case.kv_fused)
    k = dev(case.k_bits.view(np.int16)).view(torch.float16)
    sm = dev(case.slot_mapping)
    b.calls = lambda s: [pa.prepare_kv_insert_mxfp4(kv, k, sm, stream=s)]
    b.extra = {"query_tokens": T, "kv_tokens": T}
    b.config = {"workload": name, "rows": int(T), "head_dim": 128,
                "block_size": int(case.kv_fused.shape[1]), "in_dtype": "fp16",
                "sf_vec_size": 32, "slots": "random distinct, seed 1005"}
    b.dtype = "f16->mxfp4"
    b.flops = None

    def oracle_sample(n):
        import oracle

        kv_h = case.kv_fused.copy()
        oracle.mxfp4_insert(kv_h, case.k_bits[:n], case.slot_mapping[:n])
        return n / T
    b.oracle_sample = oracle_sample
    b.units = T
    b.unit_name = "rows"
    return b


def make_bench(args, torch, pa):
    import workloads as W

    name = args.workload
    if name == "fp8_decode":
        return setup_attn(args, torch, pa, W.fp8_decode(), name)
    if name == "int8_perchan":
        return setup_attn(args, torch, pa, W.int_perchan(W.KV_INT8), name)
    if name == "int4_perchan":
        return setup_attn(args, torch, pa, W.int_perchan(W.KV_INT4), name)
    if name == "fp8_verify":
        return setup_attn(args, torch, pa, W.fp8_verify(), name)
    if name == "fp8_prefill":
        return setup_attn(args, torch, pa, W.fp8_prefill(), name)
    if name == "fp8_sparse_verify":
        return setup_sparse(args, torch, pa, W.fp8_sparse_verify(), name)
    if name == "mxfp4_logits":
        return setup_logits(args, torch, pa, W.mxfp4_logits(), name)
    if name == "mxfp4_topk":
        return setup_logits(args, torch, pa, W.mxfp4_logits(), name, topk=True)
    if name == "mxfp4_insert":
        return setup_mxfp4_insert(args, torch, pa, W.mxfp4_insert_case(1005, T=32768), name)
    raise ValueError(name)


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def run_timed(args, torch, pa, hip, calls):
    """Wall-clock steps (the prepared calls rotated), with events on the
    dominant kernel's dispatch of every event_every-th launch."""
    n = len(calls)
    for k in range(args.warmup):
        calls[k % n]()
    torch.cuda.synchronize()
    every = max(1, args.event_every)
    sampled = [k for k in range(args.steps) if k % every == 0]
    evs = {k: (hip.event(), hip.event()) for k in sampled}
    torch.cuda.synchronize()
    set_events = pa.load().pa_set_profile_events  # raw C calls: keep the loop host-light
    t0 = time.perf_counter()
    for k in range(args.steps):
        if k in evs:
            set_events(*evs[k])
        elif k - 1 in evs:
            set_events(None, None)
        calls[k % n]()
    torch.cuda.synchronize()
    pa.pa_set_profile_events(None, None)
    wall = (time.perf_counter() - t0) / args.steps
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs.values()]
    for a, b in evs.values():
        hip.destroy(a)
        hip.destroy(b)
    return {"wall_s": wall, "kernel_s": sum(kern_ms) / len(kern_ms) / 1e3,
            "kernel_min_s": min(kern_ms) / 1e3, "kernel_samples": len(kern_ms)}


def graph_step_s(torch, bench, reps):
    """The steps captured once into a HIP graph (one call per pool, in order)
    and replayed: seconds per step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    calls = bench.calls(s.cuda_stream)
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (reps * len(calls))


def read_ceiling_gbps(torch, pa, nbytes=1 << 30, reps=10, grid=2048):
    """The device's streaming-read rate: the library's read probe over 1 GiB
    (past the 256 MB Infinity Cache), timed with events."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.empty(grid, dtype=torch.int32, device="cuda")
    lib = pa.load()
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        assert lib.pa_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), grid, stream) == 0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        lib.pa_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), grid, stream)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) / 1e3 / reps
    del src, sink
    return nbytes / dt / 1e9


def copy_ceiling_gbps(torch, nbytes=1 << 30, reps=10):
    """A plain device copy (read + write bytes), for counter calibration."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    return 2 * nbytes / dt / 1e9


def cpu_baseline(bench, budget_s):
    """The oracle (plain C, OpenMP over independent units) on a sample of the
    same workload: all of the host's processors, then one thread, each leg
    sized to about budget_s. Scaled to the bench unit: the sampled fraction of
    one call's work times its algorithmic bytes, per second."""
    import oracle

    oracle.load()
    oracle.set_threads(1)
    t = time.perf_counter()
    frac1 = bench.oracle_sample(1)
    t1 = time.perf_counter() - t
    legs = {}
    for name, threads in (("all", 0), ("single", 1)):
        oracle.set_threads(threads)
        cores = oracle.threads()
        n = max(1, min(bench.units, int(budget_s * (0.7 * cores if threads == 0 else 1) /
                                        max(t1, 1e-6))))
        reps = 1
        if threads == 1 and n == 1:
            dt, frac = t1, frac1
        else:
            t = time.perf_counter()
            frac = bench.oracle_sample(n)
            dt = time.perf_counter() - t
            # the whole workload well inside the budget: repeat it, so the
            # timing is not that of one short run
            if n == bench.units and dt < budget_s / 4:
                reps = 1 + int(budget_s / 4 / max(dt, 1e-6))
                t = time.perf_counter()
                for _ in range(reps - 1):
                    bench.oracle_sample(n)
                dt += time.perf_counter() - t
        legs[name] = {"value": round(reps * frac * bench.alg_bytes / dt / 1e9, 4), "unit": "GB/s",
                      "cores": cores, "kind": "oracle",
                      "sample": f"first {n} of {bench.units} {bench.unit_name} "
                                f"({100 * frac:.2f}% of one call's work)"
                                + (f", {reps} times" if reps > 1 else "") + f" in {dt:.1f} s"}
    oracle.set_threads(0)
    out = dict(legs["all"])
    out["single_thread"] = legs["single"]
    return out


def traffic_record(kernel_tag):
    """HBM traffic measured by rocprofv3 counters for the current kernel source,
    from profiles/traffic_<tag>.md; None if absent or taken on other source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256:\s*([0-9a-f]{16,64})", text)
    m_b = re.search(r"bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_b):
        return None
    if not source_hash(kernel_tag).startswith(m_src.group(1)):
        return None
    return float(m_b.group(1))


def kernel_sources(kernel_tag):
    """The source files a kernel is built from (its traffic record is tied to them)."""
    if kernel_tag.startswith("logits"):
        return ["pa_device.hpp", "pa_logits.hip"]
    if kernel_tag.startswith("topk"):
        return ["pa_device.hpp", "pa_topk.hip"]
    if kernel_tag.startswith("mxfp4_insert"):
        return ["pa_device.hpp", "pa_insert_mxfp4.hip"]
    return ["pa_device.hpp", "pa_attn.hpp", "pa_attn.hip", "pa_attn_e4m3.hip", "pa_attn_f16.hip",
            "pa_attn_bf16.hip", "pa_attn_int4.hip", "pa_attn_int8.hip"]


def source_hash(kernel_tag):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_attention_quantized_amd", "csrc")
    for f in kernel_sources(kernel_tag):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--event-every", type=int, default=4,
                    help="attach timing events to every n-th timed launch")
    ap.add_argument("--workload", default="fp8_decode", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work per CPU-baseline leg")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-rotate", action="store_true")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only the 1 GiB copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the single-GPU path has no collectives or sharding", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_attention_quantized_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.load()
    if args.copy_only:
        print(json.dumps({"copy_GBps": copy_ceiling_gbps(torch)}))
        return
    hip = Hip()
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    bench = make_bench(args, torch, pa)
    print("[bench] timing", file=sys.stderr, flush=True)
    calls = bench.calls(torch.cuda.current_stream().cuda_stream)
    r = run_timed(args, torch, pa, hip, calls)
    graph_s = None
    if not args.no_graph:
        print("[bench] graph replay", file=sys.stderr, flush=True)
        graph_s = graph_step_s(torch, bench, reps=max(1, args.steps // max(1, bench.npools)))
    print("[bench] read ceiling", file=sys.stderr, flush=True)
    read_gbps = read_ceiling_gbps(torch, pa)
    value = bench.alg_bytes / r["wall_s"] / 1e9
    achieved = bench.alg_bytes / r["kernel_s"] / 1e9
    traffic = traffic_record(bench.tag)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["wall_s"] * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": bench.dtype,
        "data": "synthetic", "config": bench.config,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "query_tokens_per_s": round(bench.extra["query_tokens"] / r["wall_s"], 1),
        "kv_tokens_per_s": round(bench.extra["kv_tokens"] / r["wall_s"], 1),
        "kernel_us": round(r["kernel_s"] * 1e6, 2), "kernel_launches_timed": r["kernel_samples"],
        "kernel_min_us": round(r["kernel_min_s"] * 1e6, 2),
        "graph_ms_per_step": None if graph_s is None else round(graph_s * 1e3, 4),
        "graph_value": None if graph_s is None else round(bench.alg_bytes / graph_s / 1e9, 1),
        "read_ceiling_GBps": round(read_gbps, 1),
        "kernel_pct_of_read_ceiling": round(100 * achieved / read_gbps, 2),
        "kv_pools_rotated": bench.npools,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": bench.tag,
                     "alg_bytes_per_launch": bench.alg_bytes},
    }
    if bench.flops is not None:
        # many query rows per KV token: the matrix cores bound this kernel
        tf = bench.flops / r["kernel_s"] / 1e12
        line["roofline"] = {"bound": "mfma", "achieved": round(tf, 1),
                            "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf / F16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                            "kernel": bench.tag, "alg_flops_per_launch": bench.flops,
                            "kv_GBps_per_launch": round(achieved, 1)}
    line.update({k: v for k, v in bench.extra.items() if k not in line})
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(bench, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
