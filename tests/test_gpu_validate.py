"""PA_VALIDATE=1: the device-side precondition check ("flashinfer.
fp4_paged_mqa_logits" API documentation, max_context_len parameter: optional
validation of the context lengths, skipped under graph capture).

Each violating input is built so that, were the check to let it through, the
attention or logits kernel would still only read memory that exists (a block
id past the declared num_blocks but inside the allocated cache, a context
length past max_context_len whose pages are real): the tests exercise the
check's verdict, never an out-of-range read. A rejected call must enqueue
nothing, so the NaN-filled output stays NaN.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import DevAttn, dev, say

pytestmark = pytest.mark.gpu


def base_case():
    return W.attn_case("validate", 5101, B=4, next_n=1, Hq=16, Hkv=4, D=128, bs=16,
                       lens=[300, 45, 130, 17], kv_kind=W.KV_E4M3,
                       scale_mode=W.SCALE_PER_TENSOR)


def call_attn(pa, case, *, num_blocks=None, max_context_len=None, noalloc=False):
    """paged_attn_fwd through the C ABI with the declared num_blocks /
    max_context_len overridden; returns (status, message, output)."""
    d = DevAttn(case)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    a = pa._attn_args(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, case.kv_kind,
                      d.ks, d.vs, case.k_scale_mode, case.v_scale_mode, case.softmax_scale,
                      case.causal)
    if num_blocks is not None:
        a.num_blocks = num_blocks
    if max_context_len is not None:
        a.max_context_len = max_context_len
    lib = pa.load()
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = lib.paged_attn_fwd_noalloc(ctypes.byref(a), stream)
    else:
        n = lib.paged_attn_workspace_size(ctypes.byref(a))
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        st = lib.paged_attn_fwd(ctypes.byref(a), ws.data_ptr(), n, stream)
    torch.cuda.synchronize()
    return st, lib.pa_last_error().decode(), out.cpu().numpy()


def with_spare_blocks(case, extra=8):
    """The case laid out contiguously (real pages in blocks 1..total) with
    `extra` random blocks allocated past them: a block id in (total, total +
    extra] lies past a declared num_blocks of total + 1 yet inside memory."""
    import dataclasses
    c = W.unpaged(case)
    rng = np.random.default_rng(7)
    pad = rng.integers(0, 256, (extra,) + c.k_cache.shape[1:], dtype=np.uint8)
    return dataclasses.replace(c, k_cache=np.concatenate([c.k_cache, pad]),
                               v_cache=np.concatenate([c.v_cache, pad]))


def violations():
    """(name, case, overrides, sequence the message must name)"""
    out = []
    c = base_case()
    c.block_table[2, 3] = 0  # a visible page of sequence 2 on the null block
    out.append(("null block", c, {}, 2))
    c = with_spare_blocks(base_case())
    declared = int(c.block_table.max()) + 1
    c.block_table[1, 1] = declared + 2  # past the declared num_blocks, inside the allocation
    out.append(("block id past num_blocks", c, {"num_blocks": declared}, 1))
    c = base_case()
    # sequence 0 (300 tokens, real pages) longer than the declared max_context_len
    out.append(("length past max_context_len", c, {"max_context_len": 250}, 0))
    c = base_case()
    c.context_lens[3] = -1
    out.append(("negative length", c, {}, 3))
    return out


@pytest.mark.parametrize("idx", range(4))
@pytest.mark.parametrize("noalloc", [False, True])
def test_validate_rejects_before_launch(pa, monkeypatch, idx, noalloc):
    monkeypatch.setenv("PA_VALIDATE", "1")
    name, case, over, seq = violations()[idx]
    say(f"validate {name} noalloc={noalloc}")
    st, msg, out = call_attn(pa, case, noalloc=noalloc, **over)
    assert st == 3, (name, st, msg)  # PA_ERR_PRECONDITION
    assert f"sequence {seq}" in msg, msg
    assert np.isnan(out.astype(np.float32)).all()  # nothing was enqueued


def test_validate_passes_valid_input_unchanged(pa, monkeypatch):
    case = base_case()
    say("validate: valid input")
    st0, _, plain = call_attn(pa, case)
    monkeypatch.setenv("PA_VALIDATE", "1")
    st1, _, checked = call_attn(pa, case)
    assert st0 == 0 and st1 == 0
    assert np.array_equal(checked.view(np.uint16), plain.view(np.uint16))


def test_validate_skipped_under_graph_capture(pa, monkeypatch):
    """While a stream is being captured the check (which syncs) is skipped:
    capture succeeds and replays equal the eager output."""
    monkeypatch.setenv("PA_VALIDATE", "1")
    case = base_case()
    d = DevAttn(case)
    n = pa.paged_attn_workspace_size(d.q, d.k, d.bt, case.max_context_len, case.kv_kind,
                                     case.k_scale_mode, case.v_scale_mode)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    eager = d.run(pa, workspace=ws).cpu().numpy()
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("validate: capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.paged_attn_fwd(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len,
                              kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs,
                              k_scale_mode=case.k_scale_mode, v_scale_mode=case.v_scale_mode,
                              softmax_scale=case.softmax_scale, causal=case.causal,
                              workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for k in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.view(np.uint16)), k


def test_validate_sparse_rejects_null_block(pa, monkeypatch):
    monkeypatch.setenv("PA_VALIDATE", "1")
    case = base_case()
    case.block_table[0, 2] = 0
    case, sel = W.with_selection(case, 5102, 40, window=8)
    d = DevAttn(case)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    say("validate sparse")
    with pytest.raises(pa.PaError, match="PRECONDITION"):
        pa.paged_attn_sparse(out, d.q, d.k, d.v, d.bt, d.cl, case.max_context_len, dev(sel),
                             kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


def logits_call(pa, case, *, num_blocks=None, max_context_len=None):
    out = torch.full((case.batch * case.next_n, case.max_context_len), float("nan"),
                     dtype=torch.float32, device="cuda")
    q, sfq, kv, w = dev(case.q), dev(case.sf_q), dev(case.kv_fused), dev(case.weights)
    cl, bt = dev(case.context_lens), dev(case.block_table)
    a = pa._logits_args(out, q, sfq, kv, w, cl, bt, case.max_context_len, 32)
    if num_blocks is not None:
        a.num_blocks = num_blocks
    if max_context_len is not None:
        a.max_context_len = max_context_len
    lib = pa.load()
    n = lib.paged_mqa_logits_workspace_size(ctypes.byref(a))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    st = lib.paged_mqa_logits(ctypes.byref(a), ws.data_ptr(), n,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, lib.pa_last_error().decode(), out.cpu().numpy()


def test_validate_logits(pa, monkeypatch):
    monkeypatch.setenv("PA_VALIDATE", "1")
    case = W.logits_case("vlog", 5103, B=3, next_n=2, H=16, D=128, bs=64, lens=[200, 64, 130],
                         max_context_len=256)
    say("validate logits: valid")
    st, msg, good = logits_call(pa, case)
    assert st == 0, msg
    # real blocks renumbered 1..used (table order), the rest of the pool left
    # allocated past them: an id above `used` is past a declared num_blocks of
    # used + 1 yet inside memory
    import dataclasses
    bt = case.block_table.copy()
    used = bt[bt > 0]
    remap = np.zeros(case.kv_fused.shape[0], np.int64)
    remap[used] = np.arange(1, used.size + 1)
    kv = case.kv_fused.copy()
    kv[1:used.size + 1] = case.kv_fused[used]
    case = dataclasses.replace(case, kv_fused=kv,
                               block_table=np.where(bt > 0, remap[bt], 0).astype(np.int32))
    assert case.kv_fused.shape[0] > used.size + 2
    case.block_table[2, 1] = used.size + 2
    say("validate logits: block id")
    st, msg, out = logits_call(pa, case, num_blocks=used.size + 1)
    assert st == 3 and "sequence 2" in msg, msg
    assert np.isnan(out).all()
    case = W.logits_case("vlog2", 5104, B=2, next_n=1, H=16, D=128, bs=64, lens=[200, 64],
                         max_context_len=256)
    say("validate logits: length")
    st, msg, out = logits_call(pa, case, max_context_len=192)
    assert st == 3 and "sequence 0" in msg, msg
    assert np.isnan(out).all()
