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
    """Device copies of an AttnCase (q as bf16 when bf16=True)."""

    def __init__(self, case: W.AttnCase, bf16=False):
        self.case = case
        self.bf16 = bf16
        self.q = dev(case.q)
        if bf16:
            self.q = self.q.to(torch.bfloat16)
        self.k = dev(case.k_cache)
        self.v = dev(case.v_cache)
        self.bt = dev(case.block_table)
        self.cl = dev(case.context_lens)
        self.ks = None if case.k_scale is None else dev(case.k_scale)
        self.vs = None if case.v_scale is None else dev(case.v_scale)

    def run(self, pa, out=None, workspace=None):
        c = self.case
        if out is None:
            out = torch.full(c.q.shape, float("nan"), dtype=self.q.dtype, device="cuda")
        pa.paged_attn_fwd(out, self.q, self.k, self.v, self.bt, self.cl, c.max_context_len,
                          kv_kind=c.kv_kind, k_scale=self.ks, v_scale=self.vs,
                          k_scale_mode=c.k_scale_mode, v_scale_mode=c.v_scale_mode,
                          softmax_scale=c.softmax_scale, causal=c.causal, workspace=workspace)
        torch.cuda.synchronize()
        return out


def to_f64(out):
    """A device output (fp16 or bf16) as float64 numpy."""
    return out.float().cpu().numpy().astype(np.float64)


def run_attn(pa, case):
    return DevAttn(case).run(pa).cpu().numpy()


def oracle_attn(case, conditioning=False, q=None):
    return oracle.paged_attn(case.q if q is None else q, case.k_cache, case.v_cache,
                             case.kv_kind, case.block_table, case.context_lens,
                             conditioning=conditioning, **case.oracle_kwargs())


def fp16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - 10)


def bf16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def attn_tolerance(ref, out_dtype="f16"):
    """max abs error 2e-3 on fp16 / bf16 outputs, widened to one ulp of the
    output type at the reference value where one ulp exceeds 2e-3 (|ref| >= 4
    for fp16, >= 0.25 for bf16): a correctly rounded output cannot be closer
    than half an ulp."""
    ulp = bf16_ulp(ref) if out_dtype == "bf16" else fp16_ulp(ref)
    return np.maximum(2e-3, ulp)


def compare_attn(got16, ref64, name, allow_rows=None, out_dtype="f16"):
    """got16: fp16 GPU output (numpy float16, or float64 values of a bf16
    output with out_dtype="bf16"); ref64: oracle float64. Returns max error / tol."""
    got = got16.astype(np.float64)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU output"
    tol = attn_tolerance(ref64, out_dtype)
    err = np.abs(got - ref64)
    bad = err > tol
    if allow_rows is not None:
        bad &= ~allow_rows[..., None]
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} elements beyond tolerance, e.g. "
                             f"{[(tuple(i), got[tuple(i)], ref64[tuple(i)]) for i in idx]}")
    return float((err / tol).max())


ILL_FACTOR = 8.0  # the conditioning margin: 8 x the fp32 score-error bound


def compare_attn_conditioned(got, ref64, cond, vrange, name, out_dtype="f16"):
    """The tolerance check with a conditioning classification.

    From the oracle (fp64): eps, a bound on the error of any fp32 evaluation
    of a row's scores; the top-2 score gap; sens[d] = sum_t p_t |V_t[d] -
    out[d]| / l, so that score errors of at most eps move out[d] by at most
    eps * sens[d] to first order.

    * An element is ill-conditioned when ILL_FACTOR * eps * sens exceeds the
      tolerance: there fp32 rounding of the scores alone can decide the
      result at the tolerance's level, whatever the kernel does. Rows whose
      top-2 gap is below ILL_FACTOR * eps (near ties, the argmax-sensitive
      case) are counted as such too.
    * Every other element must meet the tolerance.
    * An ill-conditioned element must meet tol + 2 * eps * sens (the
      first-order bound, doubled for the second order) while
      ILL_FACTOR * eps < 1 logit; beyond that (near one-hot rows with huge
      scores) it must lie within the range of V over the tokens that can carry
      weight (vrange), widened by the tolerance.

    Returns a dict of counts and the worst error / bound per class."""
    got = got.astype(np.float64)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU output"
    tol = attn_tolerance(ref64, out_dtype)
    err = np.abs(got - ref64)
    eps = cond[..., 1][..., None]
    near_tie = cond[..., 0] < ILL_FACTOR * cond[..., 1]  # [B, N, Hq]
    sens = vrange[..., 2, :]
    ill = ILL_FACTOR * eps * sens > tol
    linear = ill & (ILL_FACTOR * eps < 1.0)
    hull = ill & ~linear
    held_bad = (err > tol) & ~ill
    if held_bad.any():
        idx = np.argwhere(held_bad)[:5]
        raise AssertionError(
            f"{name}: {held_bad.sum()} elements beyond tolerance, e.g. "
            f"{[(tuple(i), got[tuple(i)], ref64[tuple(i)], cond[tuple(i[:3])], sens[tuple(i)]) for i in idx]}")
    bound = tol + 2.0 * eps * sens
    lin_bad = linear & (err > bound)
    if lin_bad.any():
        idx = np.argwhere(lin_bad)[:5]
        raise AssertionError(f"{name}: {lin_bad.sum()} ill-conditioned elements beyond the "
                             f"first-order bound, e.g. {[tuple(i) for i in idx]}")
    lo, hi = vrange[..., 0, :], vrange[..., 1, :]
    out_hull = hull & ((got < lo - tol) | (got > hi + tol))
    if out_hull.any():
        idx = np.argwhere(out_hull)[:5]
        raise AssertionError(f"{name}: {out_hull.sum()} ill-conditioned elements outside the "
                             f"V range of the tokens that can carry weight, e.g. "
                             f"{[tuple(i) for i in idx]}")
    held = ~ill
    return {"rows": int(near_tie.size), "near_tie_rows": int(near_tie.sum()),
            "elements": int(err.size), "ill_elements": int(ill.sum()),
            "ill_beyond_tol": int((ill & (err > tol)).sum()),
            "hull_checked": int(hull.sum()),
            "max_err_over_tol_held": float((err / tol)[held].max()) if held.any() else 0.0,
            "max_err_over_tol_ill": float((err / tol)[ill].max()) if ill.any() else 0.0,
            "max_err_over_bound_linear": float((err / bound)[linear].max())
            if linear.any() else 0.0}


def log_parity(record):
    """Append one parity record (a dict) to $PA_PARITY_LOG, if set."""
    import json
    import os
    path = os.environ.get("PA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")
