"""GPU parity of kv_insert_mxfp4 against the oracle, through the C ABI: the
kv_fused bytes (FP4 codes and UE8M0 scale bytes, "flashinfer.fp4_paged_mqa_logits"
API page: kv_fused, is_kv_sf_interleaved) are compared byte for byte, including
the bytes of rows without a slot, which must keep the 0xFF prefill. Then the
inserted cache is read back by paged_mqa_logits and compared bit for bit with
the oracle's logits of the oracle's cache.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


def gpu_insert(pa, case):
    kv = dev(case.kv_fused)
    dt = torch.bfloat16 if case.in_dtype == "bf16" else torch.float16
    k = dev(case.k_bits.view(np.int16)).view(dt)
    pa.kv_insert_mxfp4(kv, k, dev(case.slot_mapping), sf_interleaved=case.sf_interleaved)
    torch.cuda.synchronize()
    return kv.cpu().numpy()


def oracle_insert(case):
    kv = case.kv_fused.copy()
    return oracle.mxfp4_insert(kv, case.k_bits, case.slot_mapping, in_dtype=case.in_dtype,
                               sf_interleaved=case.sf_interleaved)


CASES = [
    dict(seed=3001, T=1000, in_dtype="f16"),
    dict(seed=3002, T=777, in_dtype="bf16", spread=40.0),
    dict(seed=3003, T=513, in_dtype="f16", sf_interleaved=True, slotless_tail=9, neg_slots=17),
    dict(seed=3004, T=300, in_dtype="bf16", sf_interleaved=True, slotless_tail=1, neg_slots=1,
         spread=100.0),
    dict(seed=3005, T=64, in_dtype="f16", spread=14.0),  # fp16 subnormals and near-max rows
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_mxfp4_insert_bit_exact(pa, idx):
    case = W.mxfp4_insert_case(**CASES[idx])
    say(f"mxfp4 insert {CASES[idx]}")
    got = gpu_insert(pa, case)
    ref = oracle_insert(case)
    diff = np.flatnonzero(got.ravel() != ref.ravel())
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:5]}"


def test_mxfp4_insert_skips_slots_outside_the_cache(pa):
    case = W.mxfp4_insert_case(3006, T=40)
    nb, bs = case.kv_fused.shape[:2]
    far = case.slot_mapping.copy()
    far[[3, 7]] = nb * bs + np.array([0, 5])  # past the last block
    case_far = W.Mxfp4InsertCase(k_bits=case.k_bits, in_dtype=case.in_dtype, slot_mapping=far,
                                 kv_fused=case.kv_fused, sf_interleaved=False)
    say("mxfp4 insert with slots past the cache")
    got = gpu_insert(pa, case_far)
    inside = far.copy()
    inside[[3, 7]] = -1
    ref = oracle_insert(W.Mxfp4InsertCase(k_bits=case.k_bits, in_dtype=case.in_dtype,
                                          slot_mapping=inside, kv_fused=case.kv_fused,
                                          sf_interleaved=False))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("interleaved", [False, True])
def test_insert_then_logits(pa, interleaved):
    """Rows inserted on the GPU, then scored by paged_mqa_logits on the GPU,
    equal the oracle's insert scored by the oracle's logits, bit for bit."""
    rng = np.random.default_rng(3007)
    T, bs = 700, 64
    case = W.mxfp4_insert_case(3007, T=T, in_dtype="bf16", sf_interleaved=interleaved, spread=3.0)
    case.slot_mapping[:] = np.arange(bs, bs + T)  # one sequence, blocks 1.. in order
    L = T
    nb = case.kv_fused.shape[0]
    cols = -(-L // 128) * 128 // bs
    bt = np.zeros((1, cols), np.int32)
    bt[0, :-(-L // bs)] = np.arange(1, 1 + -(-L // bs))
    assert bt.max() < nb
    lcase = W.logits_case("ins", 3008, B=1, next_n=2, H=64, D=128, bs=bs, lens=[L],
                          max_context_len=L)
    say(f"insert then logits, interleaved={interleaved}")
    kv_gpu = gpu_insert(pa, case)
    kv_ref = oracle_insert(case)
    assert np.array_equal(kv_gpu, kv_ref)
    out = torch.full((2, L), float("nan"), dtype=torch.float32, device="cuda")
    pa.paged_mqa_logits(dev(lcase.q), dev(lcase.sf_q), dev(kv_gpu), dev(lcase.weights),
                        dev(np.array([L], np.int32)), dev(bt), L, out=out,
                        sf_interleaved=interleaved)
    torch.cuda.synchronize()
    ref = oracle.mqa_logits(lcase.q, lcase.sf_q, kv_ref, lcase.weights, np.array([L], np.int32),
                            bt, L, sf_interleaved=interleaved)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_mxfp4_insert_errors(pa):
    kv = torch.zeros((4, 64, 1, 68), dtype=torch.uint8, device="cuda")
    k = torch.zeros((3, 128), dtype=torch.float32, device="cuda")
    sm = torch.zeros(3, dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PaError, match="UNSUPPORTED"):
        pa.kv_insert_mxfp4(kv, k, sm)
    k64 = torch.zeros((3, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(pa.PaError, match="UNSUPPORTED"):
        pa.kv_insert_mxfp4(kv, k64, sm)
