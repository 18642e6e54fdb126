"""CPU oracle for paged attention over a quantized KV cache, the MXFP4 paged MQA
logits and the KV insert.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``paged_attention_quantized_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc into
``liboracle.so``); this module only marshals numpy arrays through ctypes.
Every function's docstring names the passage of the pages it follows; the C
source carries the same citations.

Parity-pin status: every function here is pinned by tests under ``-m "not gpu"``
(see tests/test_oracle_*.py); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KV_F16, KV_BF16, KV_E4M3, KV_INT8, KV_INT4 = 0, 1, 2, 3, 4
SCALE_NONE, SCALE_PER_TENSOR, SCALE_PER_CHANNEL = 0, 1, 2

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
          "-fPIC"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (ISO C11, no FP contraction, OpenMP over
    independent units)."""
    subprocess.run(["gcc", *CFLAGS, src, "-o", out, "-lm"], check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load liboracle.so, building it first if it is not there."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = f32
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = f32
    lib.orc_f64_to_f16.argtypes = [ctypes.c_double]
    lib.orc_f64_to_f16.restype = ctypes.c_uint16
    lib.orc_f32_to_bf16.argtypes = [f32]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_to_f32.restype = f32
    lib.orc_f32_to_e4m3.argtypes = [f32]
    lib.orc_f32_to_e4m3.restype = ctypes.c_uint8
    lib.orc_round_clamp.argtypes = [f32, i32]
    lib.orc_round_clamp.restype = i32
    lib.orc_int4_value.argtypes = [i32]
    lib.orc_int4_value.restype = i32
    lib.orc_e2m1_to_f32.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_to_f32.restype = f32
    lib.orc_ue8m0_to_f32.argtypes = [ctypes.c_uint8]
    lib.orc_ue8m0_to_f32.restype = f32
    lib.orc_dequantize.argtypes = [i32, P, i64, P, i32, i64, P]
    lib.orc_dequantize.restype = None
    lib.orc_set_threads.argtypes = [i32]
    lib.orc_set_threads.restype = None
    lib.orc_threads.argtypes = []
    lib.orc_threads.restype = i32
    lib.orc_paged_attn.argtypes = [P, P, i32, P, P, i32, P, i32, P, i32, P, P,
                                   i32, i32, i32, i32, i32, i32, i64, i32, f32, i32, P, P]
    lib.orc_paged_attn.restype = i32
    lib.orc_paged_attn_sparse.argtypes = [P, P, i32, P, P, i32, P, i32, P, i32, P, P, P, i32,
                                          i32, i32, i32, i32, i32, i32, i64, i32, f32, P, P]
    lib.orc_paged_attn_sparse.restype = i32
    lib.orc_sparse_plan.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32]
    lib.orc_sparse_plan.restype = i32
    lib.orc_mqa_logits.argtypes = [P, i64, P, P, P, P, P, P,
                                   i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.orc_topk_select.argtypes = [P, P, i32, i64, P, i32, i32, i32]
    lib.orc_topk_select.restype = i32
    lib.orc_f32_to_bf16_array.argtypes = [P, P, i64]
    lib.orc_f32_to_bf16_array.restype = None
    lib.orc_f32_to_e2m1.argtypes = [f32]
    lib.orc_f32_to_e2m1.restype = ctypes.c_uint8
    lib.orc_mx_scale_byte.argtypes = [f32]
    lib.orc_mx_scale_byte.restype = ctypes.c_uint8
    lib.orc_mxfp4_insert.argtypes = [P, P, i32, P, i64, i64, i32, i32, i64, i32, i32]
    lib.orc_mxfp4_insert.restype = i32
    lib.orc_mqa_logits.restype = i32
    lib.orc_kv_insert.argtypes = [P, P, i32, P, P, i32, P, i64, i64,
                                  i32, i32, i32, i64, P, i32, P, i32]
    lib.orc_kv_insert.restype = i32
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _bits16(a):
    """fp16 / bf16 arrays may arrive as float16 or as raw uint16 bits."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint16)


# ---------------------------------------------------------------------------
# codecs (vectorised over numpy arrays by calling the scalar C routines)
# ---------------------------------------------------------------------------

def e4m3_to_f32(codes, lib=None):
    lib = lib or load()
    return np.array([lib.orc_e4m3_to_f32(int(c)) for c in np.ravel(codes)],
                    dtype=np.float32).reshape(np.shape(codes))


def f32_to_e4m3(x, lib=None):
    lib = lib or load()
    return np.array([lib.orc_f32_to_e4m3(float(v)) for v in np.ravel(np.float32(x))],
                    dtype=np.uint8).reshape(np.shape(x))


def f64_to_f16(x, lib=None):
    lib = lib or load()
    return np.array([lib.orc_f64_to_f16(float(v)) for v in np.ravel(x)],
                    dtype=np.uint16).reshape(np.shape(x)).view(np.float16)


def dequantize(kind, codes, n, scale=None, mode=SCALE_NONE, channels=1, lib=None):
    """Element-wise dequantization of a flat code array: fp32(code) * fp32(scale)."""
    lib = lib or load()
    codes = np.ascontiguousarray(codes).view(np.uint8)
    scale = _c(scale if scale is not None else np.ones(1, np.float32), np.float32)
    out = np.empty(n, np.float32)
    lib.orc_dequantize(kind, _ptr(codes), n, _ptr(scale), mode, channels, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# the three operations
# ---------------------------------------------------------------------------

def set_threads(n, lib=None):
    """Threads of the oracle's parallel loops (n <= 0: one per processor)."""
    (lib or load()).orc_set_threads(int(n))


def threads(lib=None):
    return (lib or load()).orc_threads()


def _q16(q):
    """fp16 / bf16 query bits and whether they are bf16 (a torch bfloat16
    tensor, or uint16 bits marked by the caller)."""
    try:
        import torch
        if isinstance(q, torch.Tensor):
            bf = q.dtype == torch.bfloat16
            return q.contiguous().view(torch.int16).numpy().view(np.uint16), bf
    except ImportError:  # pragma: no cover
        pass
    return _bits16(q), False


def paged_attn(q, k_cache, v_cache, kv_kind, block_table, context_lens, *,
               k_scale=None, k_scale_mode=SCALE_NONE, v_scale=None, v_scale_mode=SCALE_NONE,
               num_kv_heads, head_dim, block_size, softmax_scale, causal=True, q_is_bf16=None,
               conditioning=False, lib=None):
    """Reference paged attention (see orc_paged_attn in oracle.c).

    q: [B, next_n, Hq, D] fp16 (numpy float16 or uint16 bits), or bf16 (a torch
    bfloat16 tensor, or uint16 bits with q_is_bf16=True); caches: uint8/fp16
    arrays of shape [num_blocks, block_size, Hkv, D_bytes]. Returns float64
    [B, next_n, Hq, D]; with conditioning=True also (cond float64 [B, next_n,
    Hq, 3]: top-2 score gap, fp32 score-error bound, tokens in the relevant
    set; vrange float64 [B, next_n, Hq, 3, D]: min and max of V over that set,
    and sum_t p_t |V_t - out| / l per channel, the output's first-order
    sensitivity to score errors).
    """
    lib = lib or load()
    q16, bf = _q16(q)
    if q_is_bf16 is not None:
        bf = bool(q_is_bf16)
    B, next_n, Hq, D = q16.shape
    assert D == head_dim
    kc = np.ascontiguousarray(k_cache).view(np.uint8)
    vc = np.ascontiguousarray(v_cache).view(np.uint8)
    num_blocks = k_cache.shape[0]
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    ks = _c(k_scale if k_scale is not None else np.ones(1, np.float32), np.float32)
    vs = _c(v_scale if v_scale is not None else np.ones(1, np.float32), np.float32)
    out = np.empty((B, next_n, Hq, D), np.float64)
    cond = np.empty((B, next_n, Hq, 4), np.float64) if conditioning else None
    vr = np.empty((B, next_n, Hq, 3, D), np.float64) if conditioning else None
    rc = lib.orc_paged_attn(_ptr(out), _ptr(q16), int(bf), _ptr(kc), _ptr(vc), kv_kind,
                            _ptr(ks), k_scale_mode, _ptr(vs), v_scale_mode, _ptr(bt), _ptr(cl),
                            B, next_n, Hq, num_kv_heads, D, block_size, num_blocks,
                            bt.shape[1], float(softmax_scale), int(causal), _ptr(cond), _ptr(vr))
    if rc != 0:
        raise ValueError(f"orc_paged_attn failed with code {rc}")
    if conditioning:
        return out, cond[..., :3], vr
    return out


def paged_attn_sparse(q, k_cache, v_cache, kv_kind, block_table, context_lens, sel, *,
                      k_scale=None, k_scale_mode=SCALE_NONE, v_scale=None,
                      v_scale_mode=SCALE_NONE, num_kv_heads, head_dim, block_size,
                      softmax_scale, causal=None, q_is_bf16=None, conditioning=False,
                      lib=None):
    """Reference selection-driven sparse paged attention (see orc_paged_attn_sparse).

    sel: int32 [B, next_n, topk] logical token ids (entries outside [0, L_b)
    select nothing). Returns float64 [B, next_n, Hq, D] (with
    conditioning=True also cond and vrange as for paged_attn, over each row's
    selected tokens). `causal` is accepted for keyword compatibility with
    paged_attn and ignored.
    """
    lib = lib or load()
    q16, bf = _q16(q)
    if q_is_bf16 is not None:
        bf = bool(q_is_bf16)
    B, next_n, Hq, D = q16.shape
    assert D == head_dim
    sl = _c(sel, np.int32)
    assert sl.shape[:2] == (B, next_n)
    kc = np.ascontiguousarray(k_cache).view(np.uint8)
    vc = np.ascontiguousarray(v_cache).view(np.uint8)
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    ks = _c(k_scale if k_scale is not None else np.ones(1, np.float32), np.float32)
    vs = _c(v_scale if v_scale is not None else np.ones(1, np.float32), np.float32)
    out = np.empty((B, next_n, Hq, D), np.float64)
    cond = np.empty((B, next_n, Hq, 4), np.float64) if conditioning else None
    vr = np.empty((B, next_n, Hq, 3, D), np.float64) if conditioning else None
    rc = lib.orc_paged_attn_sparse(_ptr(out), _ptr(q16), int(bf), _ptr(kc), _ptr(vc), kv_kind,
                                   _ptr(ks), k_scale_mode, _ptr(vs), v_scale_mode, _ptr(bt),
                                   _ptr(cl), _ptr(sl), sl.shape[2], B, next_n, Hq, num_kv_heads,
                                   D, block_size, k_cache.shape[0], bt.shape[1],
                                   float(softmax_scale), _ptr(cond), _ptr(vr))
    if rc != 0:
        raise ValueError(f"orc_paged_attn_sparse failed with code {rc}")
    if conditioning:
        return out, cond[..., :3], vr
    return out


def sparse_plan(sel, block_table, context_lens, block_size, cap=None, lib=None):
    """Reference grouped union plan (see orc_sparse_plan): returns (entries int32
    [B, cap, 2] of {physical, logical block}, masks uint32 [B, cap, next_n],
    count int32 [B]); entries past count[b] are left 0."""
    lib = lib or load()
    sl = _c(sel, np.int32)
    B, next_n, topk = sl.shape
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    cap = cap or bt.shape[1]
    entries = np.zeros((B, cap, 2), np.int32)
    masks = np.zeros((B, cap, next_n), np.uint32)
    count = np.zeros(B, np.int32)
    rc = lib.orc_sparse_plan(_ptr(entries), _ptr(masks), _ptr(count), _ptr(sl), topk, _ptr(bt),
                             _ptr(cl), B, next_n, block_size, bt.shape[1], cap)
    if rc != 0:
        raise ValueError(f"orc_sparse_plan failed with code {rc}")
    return entries, masks, count


def mqa_logits(q, sf_q, kv_fused, weights, context_lens, block_table, max_context_len, *,
               sf_vec_size=32, out_rows=None, out_row_stride=None, sf_interleaved=False,
               relu=False, out_format="f32", epi_format="f32", lib=None):
    """Reference MXFP4 paged MQA logits (see orc_mqa_logits in oracle.c).

    q: uint8 [B, next_n, H, D/2]; sf_q: int32 [B, next_n, H]; kv_fused: uint8
    [num_blocks, bs, 1, D/2 + D/sf_vec] with the scale tail in token order or,
    with sf_interleaved, in the interleaved slot order; weights: fp32
    [B*next_n, H]. relu puts max(., +0) between each head's dot product and its
    weight. epi_format "f16" / "bf16" runs the weighted head chain in that type
    (see epi_step in oracle.c). Returns [B*next_n, max_context_len] (or
    [out_rows, out_row_stride])
    as fp32, or as fp16 / bf16 (uint16 bits) rounded to nearest even from the
    fp32 values for out_format "f16" / "bf16".
    """
    lib = lib or load()
    q = np.ascontiguousarray(q, np.uint8)
    B, next_n, H, Dh = q.shape
    D = Dh * 2
    bs = kv_fused.shape[1]
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    sfq = _c(sf_q, np.int32)
    w = _c(weights, np.float32)
    kv = np.ascontiguousarray(kv_fused, np.uint8)
    stride = out_row_stride or max_context_len
    rows = out_rows or B * next_n
    out = np.full((rows, stride), np.nan, np.float32)
    rc = lib.orc_mqa_logits(_ptr(out), stride, _ptr(q), _ptr(sfq), _ptr(kv), _ptr(w), _ptr(cl),
                            _ptr(bt), B, next_n, H, D, bs, bt.shape[1], max_context_len,
                            sf_vec_size, int(bool(sf_interleaved)), int(bool(relu)),
                            {"f32": 0, "f16": 1, "bf16": 2}[epi_format])
    if rc != 0:
        raise ValueError(f"orc_mqa_logits failed with code {rc}")
    if out_format == "f32":
        return out
    if out_format == "f16":
        return out.astype(np.float16)  # IEEE round to nearest even
    if out_format == "bf16":
        bits = np.empty(out.shape, np.uint16)
        lib.orc_f32_to_bf16_array(_ptr(out), _ptr(bits), out.size)
        return bits
    raise ValueError(f"unknown out_format {out_format!r}")


def topk_select(logits, context_lens, next_n, k, *, fmt="f32", lib=None):
    """Reference top-k selection (see orc_topk_select in oracle.c): logits
    [B*next_n, stride] (float32, or uint16 bits of fp16 / bf16 with fmt "f16"
    / "bf16"); returns int32 [B*next_n, k] token ids in ascending order, -1
    padded."""
    lib = lib or load()
    lg = np.ascontiguousarray(logits)
    cl = _c(context_lens, np.int32)
    rows = cl.shape[0] * next_n
    assert lg.shape[0] >= rows
    sel = np.empty((rows, k), np.int32)
    rc = lib.orc_topk_select(_ptr(sel), _ptr(lg), {"f32": 0, "f16": 1, "bf16": 2}[fmt],
                             lg.shape[1], _ptr(cl), cl.shape[0], next_n, k)
    if rc != 0:
        raise ValueError(f"orc_topk_select failed with code {rc}")
    return sel


def kv_insert(k_cache, v_cache, kv_kind, k, v, slot_mapping, *, k_scale=None,
              k_scale_mode=SCALE_NONE, v_scale=None, v_scale_mode=SCALE_NONE, in_is_bf16=False,
              block_size, lib=None):
    """Reference KV insert (see orc_kv_insert in oracle.c). Writes the caches in place."""
    lib = lib or load()
    assert k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]
    k16, v16 = _bits16(k), _bits16(v)
    T, Hkv, D = k16.shape
    sm = _c(slot_mapping, np.int64)
    ks = _c(k_scale if k_scale is not None else np.ones(1, np.float32), np.float32)
    vs = _c(v_scale if v_scale is not None else np.ones(1, np.float32), np.float32)
    rc = lib.orc_kv_insert(k_cache.ctypes.data, v_cache.ctypes.data, kv_kind, _ptr(k16),
                           _ptr(v16), int(in_is_bf16), _ptr(sm), T, sm.shape[0], Hkv, D,
                           block_size, k_cache.shape[0], _ptr(ks), k_scale_mode, _ptr(vs),
                           v_scale_mode)
    if rc != 0:
        raise ValueError(f"orc_kv_insert failed with code {rc}")


def f32_to_e2m1(x, lib=None):
    """E2M1 codes (uint8, sign in bit 3) of fp32 values, nearest-even, saturating."""
    lib = lib or load()
    return np.array([lib.orc_f32_to_e2m1(float(v)) for v in np.asarray(x, np.float32).ravel()],
                    np.uint8).reshape(np.shape(x))


def mx_scale_byte(amax, lib=None):
    """UE8M0 scale byte of a group with largest magnitude amax (see orc_mx_scale_byte)."""
    lib = lib or load()
    return np.array([lib.orc_mx_scale_byte(float(v)) for v in np.asarray(amax, np.float32).ravel()],
                    np.uint8).reshape(np.shape(amax))


def mxfp4_insert(kv_fused, k_bits, slot_mapping, *, in_dtype="f16", sf_vec_size=32,
                 sf_interleaved=False, lib=None):
    """Reference MXFP4 insert (see orc_mxfp4_insert in oracle.c): quantizes rows of
    k_bits (uint16 fp16 / bf16 bits, [T, D]) into kv_fused ([num_blocks, bs, 1,
    D/2 + D/sf_vec] uint8, modified in place) at slot_mapping (int64)."""
    lib = lib or load()
    assert kv_fused.flags.c_contiguous and kv_fused.dtype == np.uint8
    k = np.ascontiguousarray(k_bits, np.uint16)
    T, D = k.shape
    sm = _c(slot_mapping, np.int64)
    rc = lib.orc_mxfp4_insert(_ptr(kv_fused), _ptr(k), 1 if in_dtype == "bf16" else 0, _ptr(sm),
                              T, sm.shape[0], D, kv_fused.shape[1], kv_fused.shape[0],
                              sf_vec_size, int(bool(sf_interleaved)))
    if rc != 0:
        raise ValueError(f"orc_mxfp4_insert failed with code {rc}")
    return kv_fused
