"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the workload's entry point over its whole batch, inputs
resident in HBM: paged_attn_fwd (attention kernel and split merge),
paged_attn_sparse (union planner, attention, merge), paged_mqa_logits or
kv_insert_mxfp4. The default workload is
FP8 E4M3 paged decode (batch 64, 32 query / 8 KV heads, head_dim 128,
block 16, context lengths uniform in [512, 4096], seed 1001). KV pools are
replicated and rotated so consecutive steps do not hit the 256 MB Infinity
Cache. Prints one JSON line.
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
FP4_PEAK_TFLOPS = 10100.0

WORKLOADS = ("fp8_decode", "int8_perchan", "int4_perchan", "fp8_verify", "fp8_sparse_verify",
             "fp8_prefill", "mxfp4_logits", "mxfp4_insert")


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


def make_case(name):
    import workloads as W

    if name == "fp8_decode":
        return W.fp8_decode()
    if name == "int8_perchan":
        return W.int_perchan(W.KV_INT8)
    if name == "int4_perchan":
        return W.int_perchan(W.KV_INT4)
    if name == "fp8_verify":
        return W.fp8_verify()
    if name == "fp8_sparse_verify":
        return W.fp8_sparse_verify()
    if name == "fp8_prefill":
        return W.fp8_prefill()
    if name == "mxfp4_logits":
        return W.mxfp4_logits()
    if name == "mxfp4_insert":
        return W.mxfp4_insert_case(1005, T=32768, in_dtype="f16")
    raise ValueError(name)


def attn_bytes(case):
    """Algorithmic bytes of one call: K+V codes of visible tokens, the block-table
    entries of visible pages and the scales (q and out are counted apart)."""
    import workloads as W

    L = case.context_lens.astype("int64")
    kv = int(L.sum()) * case.num_kv_heads * W.row_bytes(case.kv_kind, case.head_dim) * 2
    pages = int(((L + case.block_size - 1) // case.block_size).sum())
    scales = sum(0 if s is None else s.nbytes for s in (case.k_scale, case.v_scale))
    qo = case.q.nbytes * 2
    return kv + 4 * pages + scales, qo


def attn_flops(case):
    """Matrix flops of one call: 2 D for q.k and 2 D for p.v per (query row,
    head, visible token), the visible tokens of row i being those t <= L - next_n + i
    under the causal rule (all L otherwise)."""
    import numpy as np

    L = case.context_lens.astype(np.int64)[:, None]
    i = np.arange(case.next_n, dtype=np.int64)[None, :]
    vis = np.clip(L - case.next_n + i + 1, 0, L) if case.causal else np.broadcast_to(L, (len(L), case.next_n))
    return int(vis.sum()) * case.num_q_heads * 4 * case.head_dim


def logits_bytes(case):
    L = case.context_lens.astype("int64")
    D = case.head_dim
    kv = int(L.sum()) * (D // 2 + D // 32)
    pages = int(((L + case.block_size - 1) // case.block_size).sum())
    out = case.batch * case.next_n * case.max_context_len * 4
    return kv + 4 * pages, out + case.q.nbytes + case.sf_q.nbytes + case.weights.nbytes


def copy_ceiling_gbps(torch, nbytes=1 << 30, reps=10):
    """Streaming ceiling of the box: a plain device copy (read + write bytes)."""
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
    if kernel_tag.startswith("mxfp4_insert"):
        return ["pa_device.hpp", "pa_insert_mxfp4.hip"]
    return ["pa_device.hpp", "pa_attn.hpp", "pa_attn.hip", "pa_attn_e4m3.hip", "pa_attn_f16.hip",
            "pa_attn_int4.hip", "pa_attn_int8.hip"]


def source_hash(kernel_tag):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_attention_quantized_amd", "csrc")
    for f in kernel_sources(kernel_tag):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def cpu_baseline(case, budget_s=20.0):
    """The oracle (plain C, one thread) on the first sequences of the same
    workload, scaled to the bench unit (KV GB/s)."""
    import numpy as np

    import oracle

    oracle.load()
    t_used, n_seq, kv_bytes = 0.0, 0, 0
    per_tok = None
    import workloads as W
    per_tok = case.num_kv_heads * W.row_bytes(case.kv_kind, case.head_dim) * 2
    while n_seq < case.batch and t_used < budget_s:
        sub = case.sub_batch([n_seq])
        t0 = time.perf_counter()
        oracle.paged_attn(sub.q, sub.k_cache, sub.v_cache, sub.kv_kind, sub.block_table,
                          sub.context_lens, **sub.oracle_kwargs())
        t_used += time.perf_counter() - t0
        kv_bytes += int(sub.context_lens[0]) * per_tok
        n_seq += 1
    return {"value": kv_bytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_seq} of {case.batch} sequences of the workload "
                      f"({kv_bytes / 1e6:.1f} MB of KV, {t_used:.1f} s, one thread)"}


def bench_attn(args, torch, pa, hip, case):
    import numpy as np

    alg_bytes, qo_bytes = attn_bytes(case)
    pool_bytes = case.k_cache.nbytes + case.v_cache.nbytes
    npools = max(1, math.ceil((1 << 30) / pool_bytes)) if not args.no_rotate else 1
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc = dev(case.k_cache)
    vc = dev(case.v_cache)
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(npools - 1)]
    q, bt, cl = dev(case.q), dev(case.block_table), dev(case.context_lens)
    ks = None if case.k_scale is None else dev(case.k_scale)
    vs = None if case.v_scale is None else dev(case.v_scale)
    out = torch.empty(case.q.shape, dtype=torch.float16, device="cuda")
    ws_n = pa.paged_attn_workspace_size(q, kc, bt, case.max_context_len, case.kv_kind,
                                        case.k_scale_mode, case.v_scale_mode)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    # one prepared call per pool: the timed loop only crosses the C ABI
    calls = [pa.prepare_paged_attn_fwd(out, q, kk, vv, bt, cl, case.max_context_len,
                                       kv_kind=case.kv_kind, k_scale=ks, v_scale=vs,
                                       k_scale_mode=case.k_scale_mode,
                                       v_scale_mode=case.v_scale_mode,
                                       softmax_scale=case.softmax_scale, causal=case.causal,
                                       workspace=ws, stream=stream) for kk, vv in pools]

    def step(k):
        calls[k % npools]()

    return run_timed(args, torch, pa, hip, step, alg_bytes, qo_bytes,
                     extra={"npools": npools,
                            "query_tokens": case.batch * case.next_n,
                            "kv_tokens": int(case.context_lens.astype("int64").sum())})


def sparse_bytes(case, sel):
    """Algorithmic bytes of one sparse call: K+V codes of every page in the union
    of the rows' selections (whole pages are read), the selection, and the plan
    entries and masks the attention kernel reads (q and out apart)."""
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
    plan = pages * (8 + 4 * case.next_n)
    return pages * per_page + plan + scales, case.q.nbytes * 2 + sel.nbytes, pages


def bench_sparse(args, torch, pa, hip, case_sel):
    import numpy as np

    case, sel = case_sel
    alg_bytes, other, pages = sparse_bytes(case, sel)
    pool_bytes = case.k_cache.nbytes + case.v_cache.nbytes
    npools = max(1, math.ceil((1 << 30) / pool_bytes)) if not args.no_rotate else 1
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc = dev(case.k_cache)
    vc = dev(case.v_cache)
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(npools - 1)]
    q, bt, cl, sl = dev(case.q), dev(case.block_table), dev(case.context_lens), dev(sel)
    ks = None if case.k_scale is None else dev(case.k_scale)
    vs = None if case.v_scale is None else dev(case.v_scale)
    out = torch.empty(case.q.shape, dtype=torch.float16, device="cuda")
    ws_n = pa.paged_attn_sparse_workspace_size(q, kc, bt, case.max_context_len, case.kv_kind,
                                               sel.shape[2], case.k_scale_mode,
                                               case.v_scale_mode)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    calls = [pa.prepare_paged_attn_sparse(out, q, kk, vv, bt, cl, case.max_context_len, sl,
                                          kv_kind=case.kv_kind, k_scale=ks, v_scale=vs,
                                          k_scale_mode=case.k_scale_mode,
                                          v_scale_mode=case.v_scale_mode,
                                          softmax_scale=case.softmax_scale, workspace=ws,
                                          stream=stream) for kk, vv in pools]

    def step(k):
        calls[k % npools]()

    selected = 0
    for b in range(case.batch):
        L = int(case.context_lens[b])
        for i in range(case.next_n):
            t = sel[b, i]
            selected += np.unique(t[(t >= 0) & (t < L)]).size
    return run_timed(args, torch, pa, hip, step, alg_bytes, other,
                     extra={"npools": npools, "query_tokens": case.batch * case.next_n,
                            "kv_tokens": int(selected), "union_pages": int(pages)})


def bench_logits(args, torch, pa, hip, case):
    import numpy as np

    alg_bytes, other = logits_bytes(case)
    pool_bytes = case.kv_fused.nbytes
    npools = max(1, math.ceil((1 << 30) / pool_bytes)) if not args.no_rotate else 1
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = dev(case.kv_fused)
    pools = [kv] + [kv.clone() for _ in range(npools - 1)]
    q, sfq, w = dev(case.q), dev(case.sf_q), dev(case.weights)
    cl, bt = dev(case.context_lens), dev(case.block_table)
    out = torch.empty((case.batch * case.next_n, case.max_context_len), dtype=torch.float32,
                      device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    calls = [pa.prepare_paged_mqa_logits(q, sfq, kvp, w, cl, bt, case.max_context_len, out=out,
                                         stream=stream) for kvp in pools]

    def step(k):
        calls[k % npools]()

    return run_timed(args, torch, pa, hip, step, alg_bytes + case.batch * case.next_n *
                     case.max_context_len * 4, other,
                     extra={"npools": npools, "query_tokens": case.batch * case.next_n,
                            "kv_tokens": int(case.context_lens.astype("int64").sum())})


def bench_mxfp4_insert(args, torch, pa, hip, case):
    """MXFP4 insert of T rows: algorithmic bytes are the fp16 input rows, the
    68 written bytes per row and the 8-byte slots."""
    import numpy as np

    T, D = case.k_bits.shape
    alg_bytes = T * (2 * D + D // 2 + D // 32 + 8)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = dev(case.kv_fused)
    k = dev(case.k_bits.view(np.int16)).view(torch.float16)
    sm = dev(case.slot_mapping)
    stream = torch.cuda.current_stream().cuda_stream

    call = pa.prepare_kv_insert_mxfp4(kv, k, sm, stream=stream)

    def step(_k):
        call()

    return run_timed(args, torch, pa, hip, step, alg_bytes, 0,
                     extra={"npools": 1, "query_tokens": T, "kv_tokens": T})


def run_timed(args, torch, pa, hip, step, alg_bytes, qo_bytes, extra):
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # every event_every-th launch of the timed region carries events on its
    # dominant kernel (recording them adds a few microseconds to that step)
    every = max(1, getattr(args, "event_every", 1))
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
        step(k)
    torch.cuda.synchronize()
    pa.pa_set_profile_events(None, None)
    wall = (time.perf_counter() - t0) / args.steps
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs.values()]
    for a, b in evs.values():
        hip.destroy(a)
        hip.destroy(b)
    kern_s = sum(kern_ms) / len(kern_ms) / 1e3
    return {"wall_s": wall, "kernel_s": kern_s, "kernel_min_s": min(kern_ms) / 1e3,
            "kernel_samples": len(kern_ms), "alg_bytes": alg_bytes, "qo_bytes": qo_bytes,
            **extra}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--event-every", type=int, default=4,
                    help="attach timing events to every n-th timed launch")
    ap.add_argument("--workload", default="fp8_decode", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rotate", action="store_true")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only the 1 GiB copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
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
    case = make_case(args.workload)
    print("[bench] timing", file=sys.stderr, flush=True)
    if args.workload == "mxfp4_insert":
        r = bench_mxfp4_insert(args, torch, pa, hip, case)
        tag = "mxfp4_insert"
        config = {"workload": args.workload, "rows": int(case.k_bits.shape[0]), "head_dim": 128,
                  "block_size": int(case.kv_fused.shape[1]), "in_dtype": "fp16",
                  "sf_vec_size": 32, "slots": "random distinct, seed 1005"}
        dtype = "f16->mxfp4"
    elif args.workload == "mxfp4_logits":
        r = bench_logits(args, torch, pa, hip, case)
        tag = "logits_" + args.workload
        config = {"workload": args.workload, "batch": case.batch, "next_n": case.next_n,
                  "heads": case.num_heads, "head_dim": case.head_dim,
                  "block_size": case.block_size, "max_context_len": case.max_context_len,
                  "context_lens": "uniform [1, 32768], seed 1004", "kv_dtype": "mxfp4"}
        dtype = "fp4xfp4->f32"
    elif args.workload == "fp8_sparse_verify":
        r = bench_sparse(args, torch, pa, hip, case)
        c, sel = case
        tag = "attn_ring_" + args.workload
        config = {"workload": args.workload, "batch": c.batch, "next_n": c.next_n,
                  "q_heads": c.num_q_heads, "kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                  "block_size": c.block_size, "max_context_len": c.max_context_len,
                  "kv_dtype": "e4m3", "scales": "per_tensor", "topk": 2048,
                  "selection": "last 512 tokens + uniform earlier ones per row, seed 1006",
                  "union_pages": r["union_pages"]}
        dtype = "f16xf16->f32"
    else:
        r = bench_attn(args, torch, pa, hip, case)
        # the dominant kernel: the prefill layout from 128 query rows per KV head
        rows = case.next_n * case.num_q_heads // case.num_kv_heads
        tag = ("attn_prefill_" if rows >= 128 and case.head_dim <= 128 else "attn_ring_") + \
            args.workload
        config = {"workload": args.workload, "batch": case.batch, "next_n": case.next_n,
                  "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                  "head_dim": case.head_dim, "block_size": case.block_size,
                  "max_context_len": case.max_context_len,
                  "kv_dtype": {0: "f16", 2: "e4m3", 3: "int8", 4: "int4"}[case.kv_kind],
                  "scales": {0: "none", 1: "per_tensor", 2: "per_channel"}[case.k_scale_mode],
                  "causal": bool(case.causal)}
        dtype = "f16xf16->f32"
        if case.next_n * case.num_q_heads // case.num_kv_heads > 32:
            config["row_blocks"] = -(-case.next_n * case.num_q_heads // case.num_kv_heads // 32)
    copy_gbps = copy_ceiling_gbps(torch)
    value = r["alg_bytes"] / r["wall_s"] / 1e9
    achieved = r["alg_bytes"] / r["kernel_s"] / 1e9
    traffic = traffic_record(tag)
    line = {
        "metric": "FP8-KV paged decode: effective KV GB/s and % of MI355X HBM peak; tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["wall_s"] * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic", "config": config,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "query_tokens_per_s": round(r["query_tokens"] / r["wall_s"], 1),
        "kv_tokens_per_s": round(r["kv_tokens"] / r["wall_s"], 1),
        "kernel_us": round(r["kernel_s"] * 1e6, 2), "kernel_launches_timed": r["kernel_samples"],
        "kernel_min_us": round(r["kernel_min_s"] * 1e6, 2),
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "kv_pools_rotated": r["npools"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": tag,
                     "alg_bytes_per_launch": r["alg_bytes"]},
    }
    if args.workload == "fp8_prefill":
        # many query rows per KV token: the matrix cores bound this kernel
        flops = attn_flops(case)
        tf = flops / r["kernel_s"] / 1e12
        line["roofline"] = {"bound": "mfma", "achieved": round(tf, 1),
                            "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf / F16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                            "kernel": tag, "alg_flops_per_launch": flops,
                            "kv_GBps_per_launch": round(achieved, 1)}
    if not args.no_cpu_baseline and args.workload not in ("mxfp4_logits", "mxfp4_insert",
                                                          "fp8_sparse_verify", "fp8_prefill"):
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
