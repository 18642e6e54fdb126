"""CPU checks of the C ABI: libpa.so loads, exports every function include/pa.h
declares, and the host-side argument checks return the documented status
codes without enqueuing any GPU work (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

import paged_attention_quantized_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:pa_status|size_t|const char\s*\*)\s*(\w+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("paged_attn_fwd", "paged_mqa_logits", "kv_insert", "paged_attn_workspace_size",
                 "paged_mqa_logits_workspace_size", "pa_dequantize", "pa_plan", "pa_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = pa.load()
    for name in declared_functions():
        assert hasattr(lib, name), f"libpa.so does not export {name}"
    assert set(declared_functions()) <= set(pa.EXPORTS)


def valid_args(**kw):
    fake = 0x1000  # never dereferenced: host checks reject or the call is a size query
    a = pa.AttnArgs(out=fake, q=fake, q_dtype=0, k_cache=fake, v_cache=fake, kv_kind=pa.KV_E4M3,
                    k_scale=fake, k_scale_mode=pa.SCALE_PER_TENSOR, v_scale=fake,
                    v_scale_mode=pa.SCALE_PER_TENSOR, block_table=fake, context_lens=fake,
                    max_context_len=4096, batch=64, next_n=1, num_q_heads=32, num_kv_heads=8,
                    head_dim=128, block_size=16, max_blocks_per_seq=256, num_blocks=12000,
                    softmax_scale=0.0, causal=1)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def status_of(a, ws_bytes=0):
    lib = pa.load()
    return lib.paged_attn_fwd(ctypes.byref(a), None, ws_bytes, None)


def test_workspace_size_positive_and_shape_only():
    lib = pa.load()
    n = lib.paged_attn_workspace_size(ctypes.byref(valid_args()))
    assert n > 0 and n % 256 == 0
    # independent of pointer values (device data is never read on the host)
    assert lib.paged_attn_workspace_size(ctypes.byref(valid_args(context_lens=0x2000))) == n


@pytest.mark.parametrize("field,value,status", [
    ("batch", -1, 1), ("num_kv_heads", 3, 1), ("head_dim", 100, 2), ("block_size", 8, 2),
    ("q_dtype", 2, 2), ("q_dtype", 7, 2), ("kv_kind", 9, 1), ("k_scale_mode", 7, 1), ("next_n", 0, 1),
    ("softmax_scale", -1.0, 1), ("max_blocks_per_seq", 100, 3), ("out", None, 1),
    ("k_scale", None, 1),
])
def test_host_validation(field, value, status):
    assert status_of(valid_args(**{field: value})) == status
    assert pa.load().pa_last_error().decode() != ""


def test_bf16_kinds_accepted_on_host():
    lib = pa.load()
    for kw in (dict(q_dtype=1), dict(kv_kind=pa.KV_BF16, k_scale_mode=0, v_scale_mode=0)):
        a = valid_args(**kw)
        assert lib.paged_attn_workspace_size(ctypes.byref(a)) > 0
    # a BF16 cache takes no scales
    assert status_of(valid_args(kv_kind=pa.KV_BF16)) == 2


def test_logits_workspace_holds_validation_flags():
    lib = pa.load()
    a = pa.LogitsArgs()
    assert lib.paged_mqa_logits_workspace_size(ctypes.byref(a)) == 256


def test_int4_small_head_dim_unsupported():
    a = valid_args(kv_kind=pa.KV_INT4, head_dim=64)
    assert status_of(a) == 2


def test_workspace_too_small():
    assert status_of(valid_args(), ws_bytes=16) == 4


def test_null_args():
    lib = pa.load()
    assert lib.paged_attn_fwd(None, None, 0, None) == 1
    assert lib.kv_insert(None, None) == 1
    assert lib.paged_mqa_logits(None, None, 0, None) in (1, 2)


def test_plan_info_on_host():
    lib = pa.load()
    info = (ctypes.c_int32 * 8)()
    assert lib.pa_plan(ctypes.byref(valid_args()), None, 0, None, None,
                       ctypes.cast(info, ctypes.c_void_p), None) == 0
    nwg, cap, ts, hpu, run_cost, nrb, rpb, hgroups = list(info)
    # the decode shape: one row block of 4 rows, 8 KV heads per item, 16-token items
    assert nwg >= 1 and (nrb, rpb) == (1, 4) and hpu * hgroups == 8 and ts % 16 == 0
    assert cap == 64 * nrb * hgroups * -(-4096 // ts)


def test_dequantize_validation():
    lib = pa.load()
    assert lib.pa_dequantize(9, None, 4, None, 0, 1, None, None) == 1
    assert lib.pa_dequantize(pa.KV_BF16, None, 0, None, 0, 1, None, None) == 0
    assert lib.pa_dequantize(pa.KV_E4M3, None, 3, None, 0, 1, None, None) == 1  # partial dword
    assert lib.pa_dequantize(pa.KV_E4M3, None, 0, None, 0, 1, None, None) == 0  # empty: no work


def test_insert_validation():
    lib = pa.load()
    a = pa.InsertArgs(k_cache=0x1000, v_cache=0x1000, kv_kind=pa.KV_E4M3, k=0x1000, v=0x1000,
                      in_dtype=0, slot_mapping=0x1000, num_tokens=4, num_slots=4,
                      num_kv_heads=1, head_dim=64, block_size=16, num_blocks=4,
                      k_scale=None, k_scale_mode=pa.SCALE_PER_TENSOR, v_scale=0x1000,
                      v_scale_mode=pa.SCALE_PER_TENSOR)
    assert lib.kv_insert(ctypes.byref(a), None) == 1  # scale mode set, pointer NULL
    a.num_slots = 0
    a.k_scale = 0x1000
    assert lib.kv_insert(ctypes.byref(a), None) == 0  # nothing to insert: no launch
    a.in_dtype = 1  # bf16 input into an E4M3 cache
    assert lib.kv_insert(ctypes.byref(a), None) == 0
    a.kv_kind, a.k_scale_mode, a.v_scale_mode = pa.KV_F16, 0, 0
    assert lib.kv_insert(ctypes.byref(a), None) == 2  # F16 cache needs fp16 input
    a.kv_kind = pa.KV_BF16
    assert lib.kv_insert(ctypes.byref(a), None) == 0
    a.in_dtype = 2
    assert lib.kv_insert(ctypes.byref(a), None) == 2


def test_struct_layouts_match_header(tmp_path):
    """The binding's ctypes structs have the sizes and field offsets the C
    compiler gives the structs of include/pa.h."""
    structs = {"pa_attn_args": pa.AttnArgs, "pa_logits_args": pa.LogitsArgs,
               "pa_insert_args": pa.InsertArgs, "pa_mxfp4_insert_args": pa.Mxfp4InsertArgs,
               "pa_topk_args": pa.TopkArgs}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "pa.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True,
                               text=True).stdout.split("\n"):
        if line:
            c, f, v = line.split()
            got[(c, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
