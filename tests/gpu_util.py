"""Helpers shared by the GPU parity tests: move a seeded case to the device, run
the HIP path through the C ABI, and compare with the oracle."""
import sys

import numpy as np
import torch

import oracle
import workloads as W


def say(msg):
    """Name the case before a GPU step, so a failing run shows where it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


class DevAttn:
    """Device copies of an AttnCase."""

    def __init__(self, case: W.AttnCase):
        self.case = case
        self.q = dev(case.q)
        self.k = dev(case.k_cache)
        self.v = dev(case.v_cache)
        self.bt = dev(case.block_table)
        self.cl = dev(case.context_lens)
        self.ks = None if case.k_scale is None else dev(case.k_scale)
        self.vs = None if case.v_scale is None else dev(case.v_scale)

    def run(self, pa, out=None, workspace=None):
        c = self.case
        if out is None:
            out = torch.full(c.q.shape, float("nan"), dtype=torch.float16, device="cuda")
        pa.paged_attn_fwd(out, self.q, self.k, self.v, self.bt, self.cl, c.max_context_len,
                          kv_kind=c.kv_kind, k_scale=self.ks, v_scale=self.vs,
                          k_scale_mode=c.k_scale_mode, v_scale_mode=c.v_scale_mode,
                          softmax_scale=c.softmax_scale, causal=c.causal, workspace=workspace)
        torch.cuda.synchronize()
        return out


def run_attn(pa, case):
    return DevAttn(case).run(pa).cpu().numpy()


def oracle_attn(case):
    return oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind, case.block_table,
                             case.context_lens, **case.oracle_kwargs())


def fp16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - 10)


def attn_tolerance(ref):
    """max abs error 2e-3 on fp16 outputs, widened to one fp16 ulp of the
    reference where one ulp exceeds 2e-3 (|ref| >= 4): a correctly rounded fp16
    output cannot be closer than half an ulp."""
    return np.maximum(2e-3, fp16_ulp(ref))


def compare_attn(got16, ref64, name, allow_rows=None):
    """got16: fp16 GPU output; ref64: oracle float64. Returns max error / tol."""
    got = got16.astype(np.float64)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU output"
    tol = attn_tolerance(ref64)
    err = np.abs(got - ref64)
    bad = err > tol
    if allow_rows is not None:
        bad &= ~allow_rows[..., None]
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} elements beyond tolerance, e.g. "
                             f"{[(tuple(i), got[tuple(i)], ref64[tuple(i)]) for i in idx]}")
    return float((err / tol).max())
