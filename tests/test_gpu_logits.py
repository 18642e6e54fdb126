"""GPU parity of paged_mqa_logits (MXFP4) against the oracle, through the C ABI
("flashinfer.fp4_paged_mqa_logits" API page: q, sf_q, kv_fused, weights,
context_lens, block_table, max_context_len, out).

Tolerance: max abs error <= 1e-5 on fp32 logits. With the generator's UE8M0
exponents (spread of sf_q + sf_k over a head's four 32-groups <= 8) every
per-head dot product is exact in fp32, and both sides chain the heads with
fmaf in ascending order, so the outputs are expected to be bit-identical; the
tests assert that, which implies the 1e-5 bound.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def run_gpu(pa, case, out_rows=None, out_stride=None, out_format="f32", **kw):
    rows = out_rows or case.batch * case.next_n
    stride = out_stride or case.max_context_len
    out = torch.full((rows, stride), float("nan"), dtype=TORCH_DT[out_format], device="cuda")
    pa.paged_mqa_logits(dev(case.q), dev(case.sf_q), dev(case.kv_fused), dev(case.weights),
                        dev(case.context_lens), dev(case.block_table), case.max_context_len,
                        out=out, **kw)
    torch.cuda.synchronize()
    if out_format == "bf16":
        return out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.cpu().numpy()


def run_oracle(case, out_rows=None, out_stride=None, **kw):
    return oracle.mqa_logits(case.q, case.sf_q, case.kv_fused, case.weights, case.context_lens,
                             case.block_table, case.max_context_len, out_rows=out_rows,
                             out_row_stride=out_stride, **kw)


def assert_same(got, ref, name):
    assert got.shape == ref.shape
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{name}: NaN pattern differs ({nan_g.sum()} vs {nan_r.sum()})"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isinf(got), np.isinf(ref)), f"{name}: -inf pattern differs"
    err = np.abs(got[fin].astype(np.float64) - ref[fin].astype(np.float64))
    mx = float(err.max()) if err.size else 0.0
    assert mx <= 1e-5, f"{name}: max abs error {mx}"
    same = np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert same, f"{name}: not bit-identical (max abs error {mx})"
    say(f"{name}: bit-identical, {fin.sum()} finite logits")


def small_cases():
    return [
        W.logits_case("h64_n2", 2001, B=3, next_n=2, H=64, D=128, bs=64, lens=[1, 300, 1000],
                      max_context_len=1100),
        W.logits_case("h64_n1_exact_chunks", 2002, B=3, next_n=1, H=64, D=128, bs=64,
                      lens=[64, 256, 512], max_context_len=512),
        W.logits_case("h32_n3", 2003, B=2, next_n=3, H=32, D=128, bs=64, lens=[65, 700],
                      max_context_len=777),
        W.logits_case("h16_n4", 2004, B=2, next_n=4, H=16, D=128, bs=64, lens=[255, 257],
                      max_context_len=300),
    ]


@pytest.mark.parametrize("idx", range(4))
def test_small_logits_parity(pa, idx):
    case = small_cases()[idx]
    say(f"logits parity {case.name} lens={list(case.context_lens)} max={case.max_context_len}")
    assert_same(run_gpu(pa, case), run_oracle(case), case.name)


def test_logits_untouched_rows_and_stride(pa):
    """Rows >= B*next_n and columns >= max_context_len keep their bytes; padded
    columns [L, max_context_len) hold -inf."""
    case = small_cases()[0]
    rows, stride = case.batch * case.next_n + 3, case.max_context_len + 37
    say("logits stride / untouched rows")
    got = run_gpu(pa, case, out_rows=rows, out_stride=stride)
    ref = run_oracle(case, out_rows=rows, out_stride=stride)
    assert np.isnan(got[case.batch * case.next_n:]).all()
    assert np.isnan(got[:, case.max_context_len:]).all()
    for b in range(case.batch):
        L = int(case.context_lens[b])
        for i in range(case.next_n):
            assert np.all(got[b * case.next_n + i, L:case.max_context_len] == -np.inf)
    assert_same(got, ref, "stride")


def test_logits_relocation_bit_identical(pa):
    case = small_cases()[0]
    rng = np.random.default_rng(9)
    nb = case.kv_fused.shape[0]
    perm = rng.permutation(np.arange(1, nb))
    bt = case.block_table
    remap = np.zeros(nb, np.int64)
    used = bt[bt > 0]
    remap[used] = perm[:used.size]
    kv = rng.integers(0, 256, case.kv_fused.shape, dtype=np.uint8)
    kv[0] = case.kv_fused[0]
    kv[remap[used]] = case.kv_fused[used]
    moved = dataclasses.replace(case, kv_fused=kv,
                                block_table=np.where(bt > 0, remap[bt], 0).astype(np.int32))
    say("logits relocation")
    a = run_gpu(pa, case)
    b = run_gpu(pa, moved)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_logits_errors(pa):
    case = small_cases()[0]
    out = torch.empty((case.batch * case.next_n, case.max_context_len), dtype=torch.float32,
                      device="cuda")
    narrow = dev(case.block_table[:, :2])
    with pytest.raises(pa.PaError, match="PRECONDITION"):
        pa.paged_mqa_logits(dev(case.q), dev(case.sf_q), dev(case.kv_fused), dev(case.weights),
                            dev(case.context_lens), narrow, case.max_context_len, out=out)


def test_full_mxfp4_logits(pa):
    """The full workload (B 32, next_n 2, 64 heads, lens up to 32768) in the
    launch configuration the benchmark times; every row against the oracle,
    bit for bit."""
    case = W.mxfp4_logits()
    say(f"full mxfp4 logits tokens={int(case.context_lens.sum())}")
    got = run_gpu(pa, case)
    say("full mxfp4 logits: oracle")
    assert_same(got, run_oracle(case), "full")


# ---------------------------------------------------------------------------
# API breadth ("flashinfer.fp4_paged_mqa_logits" page: output_dtype,
# is_kv_sf_interleaved; and the rectifier variant): bit-exact against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_logits_output_formats(pa, fmt):
    case = small_cases()[0]
    say(f"logits output format {fmt}")
    got = run_gpu(pa, case, out_format=fmt)
    ref = run_oracle(case, out_format=fmt)
    assert got.dtype.itemsize == 2 and ref.dtype.itemsize == 2
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), fmt


def test_logits_interleaved_scale_tail(pa):
    from tests.test_oracle_logits import interleave_sf_tail
    case = small_cases()[0]
    kv2, _ = interleave_sf_tail(case)
    inter = dataclasses.replace(case, kv_fused=kv2)
    say("logits interleaved scale tail")
    got = run_gpu(pa, inter, sf_interleaved=True)
    assert_same(got, run_oracle(inter, sf_interleaved=True), "interleaved")
    assert np.array_equal(got.view(np.uint32), run_gpu(pa, case).view(np.uint32))


@pytest.mark.parametrize("idx", [0, 2])
def test_logits_relu(pa, idx):
    case = small_cases()[idx]
    say(f"logits relu {case.name}")
    got = run_gpu(pa, case, relu=True)
    assert_same(got, run_oracle(case, relu=True), "relu " + case.name)
    plain = run_gpu(pa, case)
    assert not np.array_equal(np.nan_to_num(got), np.nan_to_num(plain))


@pytest.mark.parametrize("epi", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_logits_epilogue_types(pa, epi, fmt):
    """fp16 / bf16 epilogues (epi_dtype): the head chain in that type, bit for
    bit against the oracle's reading of it, for every output type."""
    case = small_cases()[0]
    say(f"logits epilogue {epi} out {fmt}")
    got = run_gpu(pa, case, out_format=fmt, epi_dtype=TORCH_DT[epi])
    ref = run_oracle(case, out_format=fmt, epi_format=epi)
    if fmt == "f32":
        assert_same(got, ref, f"epi {epi}")
    else:
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), (epi, fmt)


def test_logits_epilogue_full_workload(pa):
    """The full workload with an fp16 epilogue, every row bit-exact."""
    case = W.mxfp4_logits()
    say("full mxfp4 logits, fp16 epilogue")
    got = run_gpu(pa, case, epi_dtype=torch.float16)
    assert_same(got, run_oracle(case, epi_format="f16"), "full epi f16")


def test_logits_format_errors(pa):
    case = small_cases()[0]
    out = torch.empty((case.batch * case.next_n, case.max_context_len), dtype=torch.float16,
                      device="cuda")
    with pytest.raises(pa.PaError, match="INVALID_ARG"):
        pa.paged_mqa_logits(dev(case.q), dev(case.sf_q), dev(case.kv_fused), dev(case.weights),
                            dev(case.context_lens), dev(case.block_table), case.max_context_len,
                            out=out, output_dtype=torch.float32)
