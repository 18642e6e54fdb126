"""Python binding of libpa.so, the gfx950 paged-attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/pa.h. Tensors are torch tensors on the GPU (torch provides
device memory and the current stream); their data pointers are passed through.
There is no fallback: if libpa.so is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "load", "paged_attn_fwd", "paged_attn_workspace_size", "paged_attn_fwd_noalloc",
    "pa_plan", "paged_mqa_logits",
    "paged_mqa_logits_workspace_size", "kv_insert", "pa_dequantize", "pa_set_profile_events",
    "prepare_paged_attn_fwd", "prepare_paged_mqa_logits", "Prepared", "PaError",
    "kv_insert_mxfp4", "prepare_kv_insert_mxfp4",
    "KV_F16", "KV_BF16", "KV_E4M3", "KV_INT8", "KV_INT4",
    "SCALE_NONE", "SCALE_PER_TENSOR", "SCALE_PER_CHANNEL",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

DT_F16, DT_BF16, DT_F32 = 0, 1, 2
KV_F16, KV_BF16, KV_E4M3, KV_INT8, KV_INT4 = 0, 1, 2, 3, 4
SCALE_NONE, SCALE_PER_TENSOR, SCALE_PER_CHANNEL = 0, 1, 2
STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED",
          3: "PA_ERR_PRECONDITION", 4: "PA_ERR_WORKSPACE", 5: "PA_ERR_HIP"}

_vp = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class AttnArgs(ctypes.Structure):
    _fields_ = [("out", _vp), ("q", _vp), ("q_dtype", _i32), ("k_cache", _vp), ("v_cache", _vp),
                ("kv_kind", _i32), ("k_scale", _vp), ("k_scale_mode", _i32), ("v_scale", _vp),
                ("v_scale_mode", _i32), ("block_table", _vp), ("context_lens", _vp),
                ("max_context_len", _i32), ("batch", _i32), ("next_n", _i32),
                ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("max_blocks_per_seq", _i32), ("num_blocks", _i64),
                ("softmax_scale", _f32), ("causal", _i32)]


class LogitsArgs(ctypes.Structure):
    _fields_ = [("out", _vp), ("out_row_stride", _i64), ("q", _vp), ("sf_q", _vp),
                ("kv_fused", _vp), ("weights", _vp), ("context_lens", _vp), ("block_table", _vp),
                ("batch", _i32), ("next_n", _i32), ("num_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("max_blocks_per_seq", _i32), ("num_blocks", _i64),
                ("max_context_len", _i32), ("sf_vec_size", _i32), ("out_format", _i32),
                ("epi_format", _i32), ("sf_interleaved", _i32), ("relu", _i32)]


class InsertArgs(ctypes.Structure):
    _fields_ = [("k_cache", _vp), ("v_cache", _vp), ("kv_kind", _i32), ("k", _vp), ("v", _vp),
                ("in_dtype", _i32), ("slot_mapping", _vp), ("num_tokens", _i64),
                ("num_slots", _i64), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("num_blocks", _i64), ("k_scale", _vp),
                ("k_scale_mode", _i32), ("v_scale", _vp), ("v_scale_mode", _i32)]


class TopkArgs(ctypes.Structure):
    _fields_ = [("sel", _vp), ("logits", _vp), ("logits_format", _i32),
                ("logits_row_stride", _i64), ("context_lens", _vp), ("batch", _i32),
                ("next_n", _i32), ("k", _i32)]


class Mxfp4InsertArgs(ctypes.Structure):
    _fields_ = [("kv_fused", _vp), ("k", _vp), ("in_dtype", _i32), ("slot_mapping", _vp),
                ("num_tokens", _i64), ("num_slots", _i64), ("head_dim", _i32),
                ("block_size", _i32), ("num_blocks", _i64), ("sf_vec_size", _i32),
                ("sf_interleaved", _i32)]


class PaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None

EXPORTS = ["paged_attn_fwd", "paged_attn_workspace_size", "paged_attn_fwd_noalloc",
           "paged_attn_noalloc_scratch_bytes", "pa_plan", "paged_attn_sparse",
           "paged_attn_sparse_workspace_size", "pa_sparse_plan", "paged_mqa_logits",
           "paged_mqa_logits_workspace_size", "pa_topk_select", "kv_insert", "kv_insert_mxfp4",
           "pa_dequantize", "pa_read_probe",
           "pa_last_error", "pa_set_profile_events"]


def load(path: str | None = None):
    """Load libpa.so (raises if it was not built: there is no fallback path)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} not found: build it with `python -m paged_attention_quantized_amd.build`")
    lib = ctypes.CDLL(p)
    lib.paged_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), _vp, ctypes.c_size_t, _vp]
    lib.paged_attn_fwd.restype = _i32
    lib.paged_attn_workspace_size.argtypes = [ctypes.POINTER(AttnArgs)]
    lib.paged_attn_workspace_size.restype = ctypes.c_size_t
    lib.paged_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _vp]
    lib.paged_attn_fwd_noalloc.restype = _i32
    lib.paged_attn_noalloc_scratch_bytes.argtypes = []
    lib.paged_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.pa_plan.argtypes = [ctypes.POINTER(AttnArgs), _vp, _i64, _vp, _vp, _vp, _vp]
    lib.pa_plan.restype = _i32
    lib.paged_attn_sparse.argtypes = [ctypes.POINTER(AttnArgs), _vp, _i32, _vp, ctypes.c_size_t,
                                      _vp]
    lib.paged_attn_sparse.restype = _i32
    lib.paged_attn_sparse_workspace_size.argtypes = [ctypes.POINTER(AttnArgs), _i32]
    lib.paged_attn_sparse_workspace_size.restype = ctypes.c_size_t
    lib.pa_sparse_plan.argtypes = [ctypes.POINTER(AttnArgs), _vp, _i32, _vp, _vp, _vp, _i32, _vp]
    lib.pa_sparse_plan.restype = _i32
    lib.paged_mqa_logits.argtypes = [ctypes.POINTER(LogitsArgs), _vp, ctypes.c_size_t, _vp]
    lib.paged_mqa_logits.restype = _i32
    lib.paged_mqa_logits_workspace_size.argtypes = [ctypes.POINTER(LogitsArgs)]
    lib.paged_mqa_logits_workspace_size.restype = ctypes.c_size_t
    lib.pa_topk_select.argtypes = [ctypes.POINTER(TopkArgs), _vp]
    lib.pa_topk_select.restype = _i32
    lib.kv_insert.argtypes = [ctypes.POINTER(InsertArgs), _vp]
    lib.kv_insert.restype = _i32
    lib.kv_insert_mxfp4.argtypes = [ctypes.POINTER(Mxfp4InsertArgs), _vp]
    lib.kv_insert_mxfp4.restype = _i32
    lib.pa_dequantize.argtypes = [_i32, _vp, _i64, _vp, _i32, _i64, _vp, _vp]
    lib.pa_dequantize.restype = _i32
    lib.pa_read_probe.argtypes = [_vp, _i64, _vp, _i32, _vp]
    lib.pa_read_probe.restype = _i32
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_set_profile_events.argtypes = [_vp, _vp]
    lib.pa_set_profile_events.restype = _i32
    if path is None:
        _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise PaError(status, load().pa_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


class Prepared:
    """One library call with its argument struct already marshalled: calling it
    passes the same struct, workspace and stream through the C ABI again. It
    keeps references to the tensors whose pointers the struct holds."""

    def __init__(self, fn, args, keep, *rest):
        self._fn, self._args, self._ref, self._keep, self._rest = fn, args, ctypes.byref(args), \
            keep, rest

    def __call__(self):
        status = self._fn(self._ref, *self._rest)
        if status != 0:
            _check(status)


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _mode(scale, mode):
    if mode is not None:
        return mode
    if scale is None:
        return SCALE_NONE
    return SCALE_PER_TENSOR if scale.numel() == 1 else SCALE_PER_CHANNEL


# ---------------------------------------------------------------------------
# paged attention
# ---------------------------------------------------------------------------

def _need(t, name, dtypes, ndim=None, optional=False):
    """Reject a tensor the C ABI would misread: wrong dtype, rank or layout."""
    if t is None:
        if optional:
            return
        raise PaError(1, f"{name} is required")
    if t.dtype not in dtypes:
        raise PaError(1, f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise PaError(1, f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise PaError(1, f"{name} must be contiguous")


def _q_dtype(q):
    import torch
    return {torch.float16: DT_F16, torch.bfloat16: DT_BF16}[q.dtype]


def _attn_args(out, q, k_cache, v_cache, block_table, context_lens, max_context_len, kv_kind,
               k_scale, v_scale, k_scale_mode, v_scale_mode, softmax_scale, causal):
    import torch
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    _need(out, "out", (q.dtype,), 4, optional=True)
    if out is not None and out.shape != q.shape:
        raise PaError(1, f"out shape {tuple(out.shape)} != q shape {tuple(q.shape)}")
    _need(k_cache, "k_cache", (torch.uint8, torch.float16, torch.bfloat16), 4)
    _need(v_cache, "v_cache", (k_cache.dtype,), 4, optional=v_cache is None)
    _need(block_table, "block_table", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1, optional=True)
    _need(k_scale, "k_scale", (torch.float32,), optional=True)
    _need(v_scale, "v_scale", (torch.float32,), optional=True)
    B, next_n, Hq, D = q.shape
    return AttnArgs(out=_ptr(out), q=_ptr(q), q_dtype=_q_dtype(q), k_cache=_ptr(k_cache),
                    v_cache=_ptr(v_cache), kv_kind=kv_kind, k_scale=_ptr(k_scale),
                    k_scale_mode=_mode(k_scale, k_scale_mode), v_scale=_ptr(v_scale),
                    v_scale_mode=_mode(v_scale, v_scale_mode), block_table=_ptr(block_table),
                    context_lens=_ptr(context_lens), max_context_len=int(max_context_len),
                    batch=B, next_n=next_n, num_q_heads=Hq, num_kv_heads=k_cache.shape[2],
                    head_dim=D, block_size=k_cache.shape[1],
                    max_blocks_per_seq=block_table.shape[1], num_blocks=k_cache.shape[0],
                    softmax_scale=float(softmax_scale), causal=int(bool(causal)))


def paged_attn_workspace_size(q, k_cache, block_table, max_context_len, kv_kind,
                              k_scale_mode=SCALE_NONE, v_scale_mode=SCALE_NONE):
    a = _attn_args(None, q, k_cache, k_cache, block_table, None, max_context_len, kv_kind, None,
                   None, k_scale_mode, v_scale_mode, 0.0, True)
    return load().paged_attn_workspace_size(ctypes.byref(a))


def prepare_paged_attn_fwd(out, q, k_cache, v_cache, block_table, context_lens,
                           max_context_len, *, kv_kind, k_scale=None, v_scale=None,
                           k_scale_mode=None, v_scale_mode=None, softmax_scale=0.0, causal=True,
                           workspace=None, stream=None):
    """paged_attn_fwd with its argument struct built once: calling the result
    enqueues the same work again on the same tensors (their storage must stay
    alive). Arguments as for paged_attn_fwd."""
    import torch
    a = _attn_args(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                   kv_kind, k_scale, v_scale, k_scale_mode, v_scale_mode, softmax_scale, causal)
    lib = load()
    need = lib.paged_attn_workspace_size(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    return Prepared(lib.paged_attn_fwd, a, (out, q, k_cache, v_cache, workspace), _ptr(workspace),
                    workspace.numel(), _stream(stream))


def paged_attn_fwd(out, q, k_cache, v_cache, block_table, context_lens, max_context_len, *,
                   kv_kind, k_scale=None, v_scale=None, k_scale_mode=None, v_scale_mode=None,
                   softmax_scale=0.0, causal=True, workspace=None, stream=None):
    """out[B, next_n, Hq, D] <- paged attention (see paged_attn_fwd in include/pa.h).

    q fp16 or bf16 [B, next_n, Hq, D], out of q's dtype; k_cache/v_cache uint8 [num_blocks, bs, Hkv, row_bytes];
    block_table int32 [B, max_blocks]; context_lens int32 [B]; scales fp32 [1] or [Hkv, D].
    The workspace (uint8 tensor) is allocated here when not given.
    """
    prepare_paged_attn_fwd(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                           kv_kind=kv_kind, k_scale=k_scale, v_scale=v_scale,
                           k_scale_mode=k_scale_mode, v_scale_mode=v_scale_mode,
                           softmax_scale=softmax_scale, causal=causal, workspace=workspace,
                           stream=stream)()
    return out


def paged_attn_fwd_noalloc(out, q, k_cache, v_cache, block_table, context_lens,
                           max_context_len, *, kv_kind, k_scale=None, v_scale=None,
                           k_scale_mode=None, v_scale_mode=None, softmax_scale=0.0, causal=True,
                           stream=None):
    """paged_attn_fwd without a workspace: the library's own scratch array in
    device memory serves instead, and the call allocates nothing (see
    paged_attn_fwd_noalloc in include/pa.h). Arguments as for paged_attn_fwd."""
    a = _attn_args(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                   kv_kind, k_scale, v_scale, k_scale_mode, v_scale_mode, softmax_scale, causal)
    _check(load().paged_attn_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    return out


PLAN_INFO = ("workgroups", "capacity", "tokens_per_item", "heads_per_item", "run_cost",
             "row_blocks", "rows_per_block", "head_groups")


def pa_plan(block_table, context_lens, max_context_len, *, q_shape, k_cache_shape, kv_kind,
            k_scale_mode=SCALE_NONE, v_scale_mode=SCALE_NONE, causal=True, stream=None):
    """Plan probe (pa_plan in include/pa.h): returns (items int32 [total, 6] of
    {workgroup, sequence, row block, head group, first logical token, physical
    block}, seq_first int32 [B + 1], info dict)."""
    import torch
    B, next_n, Hq, D = q_shape
    nb, bs, Hkv, _ = k_cache_shape
    a = AttnArgs(q_dtype=DT_F16, kv_kind=kv_kind, k_scale_mode=k_scale_mode,
                 v_scale_mode=v_scale_mode, block_table=_ptr(block_table),
                 context_lens=_ptr(context_lens), max_context_len=int(max_context_len), batch=B,
                 next_n=next_n, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                 max_blocks_per_seq=block_table.shape[1], num_blocks=nb, softmax_scale=0.0,
                 causal=int(bool(causal)))
    lib = load()
    raw = (ctypes.c_int32 * 8)()
    _check(lib.pa_plan(ctypes.byref(a), None, 0, None, None, ctypes.cast(raw, _vp), None))
    info = dict(zip(PLAN_INFO, list(raw)))
    dev = block_table.device
    items = torch.full((max(info["capacity"], 1), 6), -1, dtype=torch.int32, device=dev)
    seq_first = torch.full((B + 1,), -1, dtype=torch.int32, device=dev)
    total = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(lib.pa_plan(ctypes.byref(a), _ptr(items), items.shape[0], _ptr(seq_first),
                       _ptr(total), ctypes.cast(raw, _vp), _stream(stream)))
    n = int(total.item())
    return items[:n], seq_first, info


# ---------------------------------------------------------------------------
# selection-driven sparse paged attention
# ---------------------------------------------------------------------------


def _sel_topk(sel, q):
    B, next_n = q.shape[0], q.shape[1]
    if sel.dim() != 3 or tuple(sel.shape[:2]) != (B, next_n):
        raise PaError(1, f"sel must be int32 [B, next_n, topk], got {tuple(sel.shape)}")
    if not sel.is_contiguous():
        raise PaError(1, "sel must be contiguous")
    return sel.shape[2]


def paged_attn_sparse_workspace_size(q, k_cache, block_table, max_context_len, kv_kind, topk,
                                     k_scale_mode=SCALE_NONE, v_scale_mode=SCALE_NONE):
    a = _attn_args(None, q, k_cache, k_cache, block_table, None, max_context_len, kv_kind, None,
                   None, k_scale_mode, v_scale_mode, 0.0, False)
    return load().paged_attn_sparse_workspace_size(ctypes.byref(a), int(topk))


def prepare_paged_attn_sparse(out, q, k_cache, v_cache, block_table, context_lens,
                              max_context_len, sel, *, kv_kind, k_scale=None, v_scale=None,
                              k_scale_mode=None, v_scale_mode=None, softmax_scale=0.0,
                              workspace=None, stream=None):
    """paged_attn_sparse with its argument struct built once (see
    prepare_paged_attn_fwd)."""
    import torch
    topk = _sel_topk(sel, q)
    a = _attn_args(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                   kv_kind, k_scale, v_scale, k_scale_mode, v_scale_mode, softmax_scale, False)
    lib = load()
    need = lib.paged_attn_sparse_workspace_size(ctypes.byref(a), topk)
    if need == 0:
        # the size query rejects these arguments: the call reports why
        _check(lib.paged_attn_sparse(ctypes.byref(a), _ptr(sel), topk, None, 0, None))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    return Prepared(lib.paged_attn_sparse, a, (out, q, k_cache, v_cache, sel, workspace),
                    _ptr(sel), topk, _ptr(workspace), workspace.numel(), _stream(stream))


def paged_attn_sparse(out, q, k_cache, v_cache, block_table, context_lens, max_context_len, sel,
                      *, kv_kind, k_scale=None, v_scale=None, k_scale_mode=None,
                      v_scale_mode=None, softmax_scale=0.0, workspace=None, stream=None):
    """out[B, next_n, Hq, D] (q's dtype) <- attention of each query row over the tokens
    it selected (sel int32 [B, next_n, topk] logical token ids; see
    paged_attn_sparse in include/pa.h). Other arguments as for paged_attn_fwd."""
    prepare_paged_attn_sparse(out, q, k_cache, v_cache, block_table, context_lens,
                              max_context_len, sel, kv_kind=kv_kind, k_scale=k_scale,
                              v_scale=v_scale, k_scale_mode=k_scale_mode,
                              v_scale_mode=v_scale_mode, softmax_scale=softmax_scale,
                              workspace=workspace, stream=stream)()
    return out


def pa_sparse_plan(sel, block_table, context_lens, max_context_len, *, q_shape, k_cache_shape,
                   kv_kind, k_scale_mode=SCALE_NONE, v_scale_mode=SCALE_NONE, cap=None,
                   stream=None):
    """Sparse planner probe: returns (entries int32 [B, cap, 2], masks int32
    [B, cap, next_n] holding the uint32 bits, count int32 [B])."""
    import torch
    B, next_n, Hq, D = q_shape
    nb, bs, Hkv, _ = k_cache_shape
    cap = int(cap or block_table.shape[1])
    a = AttnArgs(q_dtype=DT_F16, kv_kind=kv_kind, k_scale_mode=k_scale_mode,
                 v_scale_mode=v_scale_mode, block_table=_ptr(block_table),
                 context_lens=_ptr(context_lens), max_context_len=int(max_context_len), batch=B,
                 next_n=next_n, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                 max_blocks_per_seq=block_table.shape[1], num_blocks=nb, softmax_scale=0.0,
                 causal=0)
    dev = block_table.device
    entries = torch.zeros((B, cap, 2), dtype=torch.int32, device=dev)
    masks = torch.zeros((B, cap, next_n), dtype=torch.int32, device=dev)
    count = torch.zeros(B, dtype=torch.int32, device=dev)
    _check(load().pa_sparse_plan(ctypes.byref(a), _ptr(sel), sel.shape[2], _ptr(entries),
                                 _ptr(masks), _ptr(count), cap, _stream(stream)))
    return entries, masks, count


# ---------------------------------------------------------------------------
# MXFP4 paged MQA logits
# ---------------------------------------------------------------------------

LOGITS_F32, LOGITS_F16, LOGITS_BF16 = 0, 1, 2


def _logits_format(dtype):
    import torch
    formats = {torch.float32: LOGITS_F32, torch.float16: LOGITS_F16, torch.bfloat16: LOGITS_BF16}
    if dtype not in formats:
        raise PaError(1, f"logits dtype must be float32, float16 or bfloat16, got {dtype}")
    return formats[dtype]


def _logits_args(out, q, sf_q, kv_fused, weights, context_lens, block_table, max_context_len,
                 sf_vec_size, out_format=LOGITS_F32, epi_format=LOGITS_F32, sf_interleaved=False,
                 relu=False):
    B, next_n, H, Dh = q.shape
    return LogitsArgs(out=_ptr(out), out_row_stride=_row_stride(out) if out is not None else 0,
                      q=_ptr(q), sf_q=_ptr(sf_q), kv_fused=_ptr(kv_fused), weights=_ptr(weights),
                      context_lens=_ptr(context_lens), block_table=_ptr(block_table), batch=B,
                      next_n=next_n, num_heads=H, head_dim=2 * Dh, block_size=kv_fused.shape[1],
                      max_blocks_per_seq=block_table.shape[1], num_blocks=kv_fused.shape[0],
                      max_context_len=int(max_context_len), sf_vec_size=int(sf_vec_size),
                      out_format=out_format, epi_format=epi_format,
                      sf_interleaved=int(bool(sf_interleaved)), relu=int(bool(relu)))


def paged_mqa_logits_workspace_size(q, sf_q, kv_fused, weights, context_lens, block_table,
                                    max_context_len, sf_vec_size=32):
    a = _logits_args(None, q, sf_q, kv_fused, weights, context_lens, block_table,
                     max_context_len, sf_vec_size)
    return load().paged_mqa_logits_workspace_size(ctypes.byref(a))


def prepare_paged_mqa_logits(q, sf_q, kv_fused, weights, context_lens, block_table,
                             max_context_len, *, sf_vec_size=32, output_dtype=None,
                             epi_dtype=None, sf_interleaved=False, relu=False, out=None,
                             workspace=None, stream=None):
    """paged_mqa_logits with its argument struct built once (see
    prepare_paged_attn_fwd); the result's .out is the output tensor."""
    import torch
    B, next_n = q.shape[:2]
    if output_dtype is None:
        output_dtype = out.dtype if out is not None else torch.float32
    if out is None:
        out = torch.empty((B * next_n, max_context_len), dtype=output_dtype, device=q.device)
    elif out.dtype != output_dtype:
        raise PaError(1, f"out is {out.dtype} but output_dtype is {output_dtype}")
    a = _logits_args(out, q, sf_q, kv_fused, weights, context_lens, block_table,
                     max_context_len, sf_vec_size, _logits_format(output_dtype),
                     _logits_format(epi_dtype or torch.float32), sf_interleaved, relu)
    lib = load()
    need = lib.paged_mqa_logits_workspace_size(ctypes.byref(a))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    call = Prepared(lib.paged_mqa_logits, a, (out, q, kv_fused, workspace), _ptr(workspace),
                    workspace.numel() if workspace is not None else 0, _stream(stream))
    call.out = out
    return call


def paged_mqa_logits(q, sf_q, kv_fused, weights, context_lens, block_table, max_context_len, *,
                     sf_vec_size=32, output_dtype=None, epi_dtype=None, sf_interleaved=False,
                     relu=False, out=None, workspace=None, stream=None):
    """Weighted per-head MXFP4 logits [B*next_n, max_context_len] (include/pa.h):
    float32 by default, or output_dtype float16 / bfloat16; sf_interleaved
    reads kv_fused scale tails in the interleaved slot order; relu applies
    max(., 0) between each head's dot product and its weight."""
    call = prepare_paged_mqa_logits(q, sf_q, kv_fused, weights, context_lens, block_table,
                                    max_context_len, sf_vec_size=sf_vec_size,
                                    output_dtype=output_dtype, epi_dtype=epi_dtype,
                                    sf_interleaved=sf_interleaved, relu=relu, out=out,
                                    workspace=workspace, stream=stream)
    call()
    return call.out


# ---------------------------------------------------------------------------
# top-k selection: logits -> per-row token ids for paged_attn_sparse
# ---------------------------------------------------------------------------

def _row_stride(t):
    """Elements between rows of a 2-D tensor (a tensor of one row may carry
    any stride for its first dimension; its row length is used)."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def prepare_topk_select(logits, context_lens, next_n, k, *, sel=None, stream=None):
    """pa_topk_select with its argument struct built once; the result's .sel is
    the output [B*next_n, k] int32 (see pa_topk_select in include/pa.h)."""
    import torch
    _need(logits, "logits", (torch.float32, torch.float16, torch.bfloat16), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    B = context_lens.shape[0]
    if logits.shape[0] < B * next_n:
        raise PaError(1, f"logits has {logits.shape[0]} rows, needs {B * next_n}")
    if sel is None:
        sel = torch.empty((B * next_n, k), dtype=torch.int32, device=logits.device)
    _need(sel, "sel", (torch.int32,))
    a = TopkArgs(sel=_ptr(sel), logits=_ptr(logits), logits_format=_logits_format(logits.dtype),
                 logits_row_stride=_row_stride(logits), context_lens=_ptr(context_lens), batch=B,
                 next_n=int(next_n), k=int(k))
    call = Prepared(load().pa_topk_select, a, (sel, logits, context_lens), _stream(stream))
    call.sel = sel
    return call


def topk_select(logits, context_lens, next_n, k, *, sel=None, stream=None):
    """Token ids of the k largest logits per row, ascending, -1 padded:
    int32 [B*next_n, k], ready as paged_attn_sparse's sel (viewed [B, next_n, k])."""
    call = prepare_topk_select(logits, context_lens, next_n, k, sel=sel, stream=stream)
    call()
    return call.sel


# ---------------------------------------------------------------------------
# KV insert and the codec probe
# ---------------------------------------------------------------------------

def kv_insert(k_cache, v_cache, k, v, slot_mapping, *, kv_kind, k_scale=None, v_scale=None,
              k_scale_mode=None, v_scale_mode=None, stream=None):
    """Quantize rows k, v [T, Hkv, D] (fp16 or bf16) into the paged caches at
    slot_mapping (int64)."""
    import torch
    _need(k, "k", (torch.float16, torch.bfloat16), 3)
    _need(v, "v", (k.dtype,), 3)
    _need(slot_mapping, "slot_mapping", (torch.int64,), 1)
    _need(k_cache, "k_cache", (torch.uint8, torch.float16, torch.bfloat16), 4)
    _need(v_cache, "v_cache", (k_cache.dtype,), 4)
    _need(k_scale, "k_scale", (torch.float32,), optional=True)
    _need(v_scale, "v_scale", (torch.float32,), optional=True)
    T, Hkv, D = k.shape
    a = InsertArgs(k_cache=_ptr(k_cache), v_cache=_ptr(v_cache), kv_kind=kv_kind, k=_ptr(k),
                   v=_ptr(v), in_dtype=_q_dtype(k), slot_mapping=_ptr(slot_mapping),
                   num_tokens=T, num_slots=slot_mapping.shape[0], num_kv_heads=Hkv, head_dim=D,
                   block_size=k_cache.shape[1], num_blocks=k_cache.shape[0],
                   k_scale=_ptr(k_scale), k_scale_mode=_mode(k_scale, k_scale_mode),
                   v_scale=_ptr(v_scale), v_scale_mode=_mode(v_scale, v_scale_mode))
    _check(load().kv_insert(ctypes.byref(a), _stream(stream)))


def prepare_kv_insert_mxfp4(kv_fused, k, slot_mapping, *, sf_interleaved=False, stream=None):
    """kv_insert_mxfp4 with its argument struct built once (see prepare_paged_attn_fwd)."""
    import torch
    dt = {torch.float16: DT_F16, torch.bfloat16: DT_BF16}.get(k.dtype)
    if dt is None:
        raise PaError(2, f"kv_insert_mxfp4: k must be float16 or bfloat16, got {k.dtype}")
    a = Mxfp4InsertArgs(kv_fused=_ptr(kv_fused), k=_ptr(k), in_dtype=dt,
                        slot_mapping=_ptr(slot_mapping), num_tokens=k.shape[0],
                        num_slots=slot_mapping.shape[0], head_dim=k.shape[1],
                        block_size=kv_fused.shape[1], num_blocks=kv_fused.shape[0],
                        sf_vec_size=32, sf_interleaved=int(bool(sf_interleaved)))
    return Prepared(load().kv_insert_mxfp4, a, (kv_fused, k, slot_mapping), _stream(stream))


def kv_insert_mxfp4(kv_fused, k, slot_mapping, *, sf_interleaved=False, stream=None):
    """Quantize rows k [T, 128] (fp16 or bf16) to MXFP4 into kv_fused
    [num_blocks, block_size, 1, 68] uint8 at slot_mapping (int64), the layout
    paged_mqa_logits reads (include/pa.h)."""
    prepare_kv_insert_mxfp4(kv_fused, k, slot_mapping, sf_interleaved=sf_interleaved,
                            stream=stream)()


def pa_set_profile_events(start_event, stop_event):
    """Bracket the dominant kernel of later calls with two hipEvent_t handles (or clear)."""
    _check(load().pa_set_profile_events(start_event, stop_event))


def pa_dequantize(kind, codes, n, scale=None, mode=None, channels=1, out=None, stream=None):
    """Codec probe: out[i] = fp32(code_i) * scale (include/pa.h)."""
    import torch
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    _check(load().pa_dequantize(kind, _ptr(codes), n, _ptr(scale), _mode(scale, mode), channels,
                                _ptr(out), _stream(stream)))
    return out
