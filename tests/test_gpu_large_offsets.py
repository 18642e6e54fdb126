"""Caches larger than 4 GiB. Each case runs twice: on its compact cache, and on
a cache of ~4.4 GiB per plane on the device whose real pages sit at the top
physical block ids, where their byte offsets exceed 2^32. Cache addresses are
formed from 64-bit products of block id and page size, so both runs give the
same bytes: the outputs are compared bit for bit (relocation invariance), and
the compact run against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DevAttn, compare_attn, dev, say

pytestmark = pytest.mark.gpu

BIG_BYTES = int(4.4 * 2**30)  # per cache plane


def _high_ids(n_used, nb_big, page_bytes):
    """Block ids for n_used pages at the top of a cache of nb_big blocks, all
    of them starting past byte offset 2^32."""
    ids = nb_big - 1 - np.arange(n_used, dtype=np.int64)
    assert ids.min() * page_bytes >= 2**32
    return ids


def _big_plane(compact, used, ids, nb_big):
    """A device cache of nb_big blocks: block 0 (the null block) and the used
    pages copied from `compact` (numpy, [nb, ...]) to ids; the rest is left
    as allocated (never read)."""
    big = torch.empty((nb_big,) + compact.shape[1:], dtype=torch.uint8, device="cuda")
    big[0] = dev(compact[0])
    big[dev(ids)] = dev(compact[used])
    return big


def _place_high(case):
    """(k_big, v_big, block_table) of an AttnCase with its pages at high ids."""
    page = int(np.prod(case.k_cache.shape[1:]))
    nb_big = BIG_BYTES // page + 1
    bt = case.block_table
    used = np.unique(bt[bt > 0])
    ids = _high_ids(used.size, nb_big, page)
    remap = np.zeros(case.num_blocks, np.int64)
    remap[used] = ids
    bt_big = np.where(bt > 0, remap[bt], 0).astype(np.int32)
    return (_big_plane(case.k_cache, used, ids, nb_big),
            _big_plane(case.v_cache, used, ids, nb_big), bt_big)


def _attn(pa, case, k, v, bt, sel=None):
    d = DevAttn(case)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device="cuda")
    kw = dict(kv_kind=case.kv_kind, k_scale=d.ks, v_scale=d.vs, k_scale_mode=case.k_scale_mode,
              v_scale_mode=case.v_scale_mode, softmax_scale=case.softmax_scale)
    if sel is None:
        pa.paged_attn_fwd(out, d.q, k, v, dev(bt), d.cl, case.max_context_len, causal=case.causal,
                          **kw)
    else:
        pa.paged_attn_sparse(out, d.q, k, v, dev(bt), d.cl, case.max_context_len, dev(sel), **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


ATTN_CASES = [
    ("fp8_decode", dict(B=3, next_n=1, Hq=32, Hkv=8, D=128, bs=16, lens=[300, 1000, 17],
                        kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)),
    ("int4_perchan_rows", dict(B=2, next_n=2, Hq=16, Hkv=2, D=256, bs=32, lens=[700, 129],
                               kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_CHANNEL)),
    ("fp8_prefill_layout", dict(B=1, next_n=16, Hq=64, Hkv=8, D=128, bs=32, lens=[900],
                                kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)),
]


@pytest.mark.parametrize("idx", range(len(ATTN_CASES)))
def test_attention_past_4gib(pa, idx):
    name, kw = ATTN_CASES[idx]
    case = W.attn_case("big_" + name, 8101 + idx, **kw)
    say(f"past 4 GiB: {name} compact")
    base = _attn(pa, case, dev(case.k_cache), dev(case.v_cache), case.block_table)
    if case.k_scale_mode != W.SCALE_PER_CHANNEL:  # (per-channel parity: the conditioned tests)
        ref = oracle.paged_attn(case.q, case.k_cache, case.v_cache, case.kv_kind,
                                case.block_table, case.context_lens, **case.oracle_kwargs())
        compare_attn(base, ref, case.name)
    say(f"past 4 GiB: {name} high ids")
    kb, vb, bt = _place_high(case)
    got = _attn(pa, case, kb, vb, bt)
    del kb, vb
    torch.cuda.empty_cache()
    assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


def test_sparse_past_4gib(pa):
    case = W.attn_case("big_sparse", 8111, B=2, next_n=4, Hq=64, Hkv=8, D=128, bs=32,
                       lens=[1500, 600], kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    case, sel = W.with_selection(case, 8112, 256)
    say("past 4 GiB: sparse compact")
    base = _attn(pa, case, dev(case.k_cache), dev(case.v_cache), case.block_table, sel)
    say("past 4 GiB: sparse high ids")
    kb, vb, bt = _place_high(case)
    got = _attn(pa, case, kb, vb, bt, sel)
    del kb, vb
    torch.cuda.empty_cache()
    assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


def test_logits_past_4gib(pa):
    lens = np.array([2000, 333], np.int32)
    lg = W.logits_case("big_logits", 8121, B=2, next_n=2, H=64, D=128, bs=64, lens=lens,
                       max_context_len=2048)
    args = (dev(lg.q), dev(lg.sf_q))
    say("past 4 GiB: logits compact")
    base = pa.paged_mqa_logits(*args, dev(lg.kv_fused), dev(lg.weights), dev(lens),
                               dev(lg.block_table), lg.max_context_len).cpu().numpy()
    ref = oracle.mqa_logits(lg.q, lg.sf_q, lg.kv_fused, lg.weights, lens, lg.block_table,
                            lg.max_context_len)
    assert np.array_equal(base.view(np.uint32), ref.view(np.uint32))
    page = int(np.prod(lg.kv_fused.shape[1:]))
    nb_big = BIG_BYTES // page + 1
    bt = lg.block_table
    used = np.unique(bt[bt > 0])
    ids = _high_ids(used.size, nb_big, page)
    remap = np.zeros(lg.kv_fused.shape[0], np.int64)
    remap[used] = ids
    bt_big = np.where(bt > 0, remap[bt], 0).astype(np.int32)
    kv = _big_plane(lg.kv_fused, used, ids, nb_big)
    say("past 4 GiB: logits high ids")
    got = pa.paged_mqa_logits(*args, kv, dev(lg.weights), dev(lens), dev(bt_big),
                              lg.max_context_len).cpu().numpy()
    del kv
    torch.cuda.empty_cache()
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


def test_inserts_past_4gib(pa):
    """kv_insert and kv_insert_mxfp4 into slots whose byte offsets exceed 2^32
    write the same bytes as into the compact cache."""
    ins = W.insert_case(8131, T=300, Hkv=8, D=128, bs=16, kv_kind=W.KV_E4M3,
                        scale_mode=W.SCALE_PER_TENSOR, value_scale=2.0)
    k, v = dev(ins.k), dev(ins.v)
    ks, vs = dev(ins.k_scale), dev(ins.v_scale)
    kw = dict(kv_kind=ins.kv_kind, k_scale=ks, v_scale=vs, k_scale_mode=ins.scale_mode,
              v_scale_mode=ins.scale_mode)
    say("past 4 GiB: kv_insert compact")
    kc, vc = dev(ins.k_cache), dev(ins.v_cache)
    pa.kv_insert(kc, vc, k, v, dev(ins.slot_mapping), **kw)
    bs = ins.block_size
    page = int(np.prod(ins.k_cache.shape[1:]))
    nb_big = BIG_BYTES // page + 1
    blocks = np.unique(ins.slot_mapping[ins.slot_mapping >= 0] // bs)
    ids = _high_ids(blocks.size, nb_big, page)
    remap = np.zeros(ins.num_blocks, np.int64)
    remap[blocks] = ids
    sm = ins.slot_mapping.copy()
    ok = sm >= 0
    sm[ok] = remap[sm[ok] // bs] * bs + sm[ok] % bs
    say("past 4 GiB: kv_insert high slots")
    kb = torch.empty((nb_big,) + ins.k_cache.shape[1:], dtype=torch.uint8, device="cuda")
    vb = torch.empty_like(kb)
    kb[dev(ids)] = dev(ins.k_cache[blocks])
    vb[dev(ids)] = dev(ins.v_cache[blocks])
    pa.kv_insert(kb, vb, k, v, dev(sm), **kw)
    torch.cuda.synchronize()
    assert np.array_equal(kb[dev(ids)].cpu().numpy(), kc[dev(blocks)].cpu().numpy())
    assert np.array_equal(vb[dev(ids)].cpu().numpy(), vc[dev(blocks)].cpu().numpy())
    del kb, vb
    torch.cuda.empty_cache()

    mx = W.mxfp4_insert_case(8132, T=300, in_dtype="f16", spread=3.0)
    keys = dev(mx.k_bits.view(np.int16)).view(torch.float16)
    say("past 4 GiB: kv_insert_mxfp4 compact")
    kvc = dev(mx.kv_fused)
    pa.kv_insert_mxfp4(kvc, keys, dev(mx.slot_mapping))
    bs = mx.kv_fused.shape[1]
    page = int(np.prod(mx.kv_fused.shape[1:]))
    nb_big = BIG_BYTES // page + 1
    blocks = np.unique(mx.slot_mapping // bs)
    ids = _high_ids(blocks.size, nb_big, page)
    remap = np.zeros(mx.kv_fused.shape[0], np.int64)
    remap[blocks] = ids
    sm = remap[mx.slot_mapping // bs] * bs + mx.slot_mapping % bs
    say("past 4 GiB: kv_insert_mxfp4 high slots")
    kvb = torch.empty((nb_big,) + mx.kv_fused.shape[1:], dtype=torch.uint8, device="cuda")
    kvb[dev(ids)] = dev(mx.kv_fused[blocks])
    pa.kv_insert_mxfp4(kvb, keys, dev(sm))
    torch.cuda.synchronize()
    assert np.array_equal(kvb[dev(ids)].cpu().numpy(), kvc[dev(blocks)].cpu().numpy())
    del kvb
    torch.cuda.empty_cache()
