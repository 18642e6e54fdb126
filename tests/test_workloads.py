"""The seeded generators produce the shapes and structure the workloads state."""
import numpy as np

import workloads as W


def test_tiny_f16_layout():
    c = W.tiny_f16()
    assert c.q.shape == (2, 1, 4, 64) and c.q.dtype == np.float16
    assert c.k_cache.shape == (16, 16, 1, 128)
    assert list(c.context_lens) == [37, 70]
    assert c.block_table.shape == (2, 5)
    row0, row1 = c.block_table
    assert list(row0[3:]) == [0, 0] and (row0[:3] > 0).all() and (row1 > 0).all()
    used = np.concatenate([row0[:3], row1])
    assert len(set(used.tolist())) == 8 and used.min() >= 1 and used.max() <= 15
    assert c.softmax_scale == 0.125
    # null block holds fp16 NaN
    assert np.isnan(c.k_cache[0].view(np.float16)).all()


def test_generators_are_seeded():
    a, b = W.tiny_f16(), W.tiny_f16()
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.q, b.q)
    c = W.attn_case("x", 3, B=2, next_n=1, Hq=2, Hkv=1, D=16, bs=4, lens=[5, 9],
                    kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    d = W.attn_case("x", 3, B=2, next_n=1, Hq=2, Hkv=1, D=16, bs=4, lens=[5, 9],
                    kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    assert np.array_equal(c.k_cache, d.k_cache)


def test_e4m3_null_block_poison_and_scale():
    c = W.attn_case("x", 4, B=3, next_n=1, Hq=4, Hkv=2, D=32, bs=16, lens=[40, 17, 64],
                    kv_kind=W.KV_E4M3, scale_mode=W.SCALE_PER_TENSOR)
    assert set(np.unique(c.k_cache[0]).tolist()) == {0x7F, 0xFF}
    assert set(np.unique(c.v_cache[0]).tolist()) == {0x7F, 0xFF}
    # tail slots of the last page of sequence 0 (40 = 2*16 + 8) are NaN bytes
    last = c.block_table[0, 2]
    assert set(np.unique(c.k_cache[last, 8:]).tolist()) <= {0x7F, 0xFF}
    assert c.k_scale.shape == (1,) and c.k_scale[0] > 0


def test_relocate_and_unpaged_keep_logical_content():
    c = W.attn_case("x", 5, B=2, next_n=1, Hq=2, Hkv=1, D=16, bs=4, lens=[7, 12],
                    kv_kind=W.KV_INT8, scale_mode=W.SCALE_PER_TENSOR)
    for o in (W.relocate(c, 1), W.unpaged(c)):
        for b in range(2):
            n = -(-int(c.context_lens[b]) // 4)
            assert np.array_equal(o.k_cache[o.block_table[b, :n]], c.k_cache[c.block_table[b, :n]])
            assert np.array_equal(o.v_cache[o.block_table[b, :n]], c.v_cache[c.block_table[b, :n]])
    r = W.relocate(c, 1)
    assert not np.array_equal(r.block_table, c.block_table)


def test_per_channel_recipe():
    c = W.attn_case("x", 6, B=1, next_n=1, Hq=4, Hkv=2, D=32, bs=8, lens=[30],
                    kv_kind=W.KV_INT4, scale_mode=W.SCALE_PER_CHANNEL, zero_k_channel_frac=0.1,
                    q_dist=(-100.0, 100.0))
    assert c.k_scale.shape == (2, 32) and c.k_scale.min() >= 1e-2 and c.k_scale.max() <= 1e3
    assert c.k_cache.shape[-1] == 16
    assert np.abs(c.q.astype(np.float32)).max() <= 100.0


def test_logits_layout():
    c = W.logits_case("l", 2, B=2, next_n=2, H=4, D=128, bs=64, lens=[257, 3],
                      max_context_len=300)
    assert c.kv_fused.shape[1:] == (64, 1, 68)
    assert c.block_table.shape == (2, 6)
    assert c.sf_q.dtype == np.int32 and c.sf_q.shape == (2, 2, 4)
    assert (c.kv_fused[0].reshape(-1)[64 * 64:] == 0xFF).all()  # null block SF poisoned
