"""Seeded synthetic inputs for paged attention, MXFP4 paged MQA logits and the
KV insert.

This module is shared by the oracle-side tests and the GPU-side tests and
benchmark, and holds none of the method's arithmetic: integer and FP4 codes
are drawn directly, and FP8 E4M3 codes for normally distributed values come
from torch's own ``float8_e4m3fn`` cast (a library conversion, not this
project's codec). Every array is numpy; callers move them to the device.

Workloads (sizes as the pages' benchmark configurations fix them):
  tiny_f16      B 2, 1 row, 4 q heads / 1 KV head, D 64, block 16, lens {37, 70}
  fp8_decode    B 64, 1 row, 32/8 heads, D 128, block 16, lens U[512, 4096], E4M3 per tensor
  int_perchan   B 32, 1 row, 16/2 heads, D 256, block 32, len 8192, INT4 or INT8 per channel
  fp8_verify    B 16, 4 rows causal, 64/8 heads, D 128, block 32, lens U[4096, 16384], E4M3
  mxfp4_logits  B 32, next_n 2, 64 heads, D 128, block 64, lens U[1, 32768]
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

KV_F16, KV_BF16, KV_E4M3, KV_INT8, KV_INT4 = 0, 1, 2, 3, 4
SCALE_NONE, SCALE_PER_TENSOR, SCALE_PER_CHANNEL = 0, 1, 2

SEED_BASE = 1000  # workload k (0..4) uses numpy default_rng(1000 + k)


def row_bytes(kind: int, D: int) -> int:
    return {KV_F16: 2 * D, KV_BF16: 2 * D, KV_E4M3: D, KV_INT8: D, KV_INT4: D // 2}[kind]


def e4m3_codes_torch(x: np.ndarray) -> np.ndarray:
    """FP8 E4M3 codes of fp32 values via torch's float8_e4m3fn cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclasses.dataclass
class AttnCase:
    name: str
    q: np.ndarray  # float16 [B, next_n, Hq, D]
    k_cache: np.ndarray  # uint8 [num_blocks, bs, Hkv, row_bytes]
    v_cache: np.ndarray
    kv_kind: int
    k_scale: np.ndarray | None  # float32 [1] or [Hkv, D]
    v_scale: np.ndarray | None
    k_scale_mode: int
    v_scale_mode: int
    block_table: np.ndarray  # int32 [B, max_blocks]
    context_lens: np.ndarray  # int32 [B]
    max_context_len: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    softmax_scale: float
    causal: bool

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def next_n(self):
        return self.q.shape[1]

    @property
    def num_q_heads(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    def oracle_kwargs(self):
        return dict(k_scale=self.k_scale, k_scale_mode=self.k_scale_mode, v_scale=self.v_scale,
                    v_scale_mode=self.v_scale_mode, num_kv_heads=self.num_kv_heads,
                    head_dim=self.head_dim, block_size=self.block_size,
                    softmax_scale=self.softmax_scale, causal=self.causal)

    def kv_bytes_visible(self) -> int:
        """K+V code bytes of visible tokens (each token is visible to some row)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * \
            row_bytes(self.kv_kind, self.head_dim) * 2

    def sub_batch(self, idx):
        """Same caches, only sequences idx (for sampled checks at full size)."""
        idx = np.asarray(idx)
        return dataclasses.replace(self, q=self.q[idx], block_table=self.block_table[idx],
                                   context_lens=self.context_lens[idx])


def _poison_byte_pattern(kind: int, n: int, rng) -> np.ndarray:
    """Bytes that decode to NaN where the format has NaN (E4M3 0x7F/0xFF,
    fp16 0x7E00), random bytes otherwise."""
    if kind == KV_E4M3:
        return np.where(np.arange(n) % 2 == 0, 0x7F, 0xFF).astype(np.uint8)
    if kind == KV_F16:
        return np.tile(np.array([0x00, 0x7E], np.uint8), n // 2 + 1)[:n]
    if kind == KV_BF16:
        return np.tile(np.array([0xC0, 0x7F], np.uint8), n // 2 + 1)[:n]
    return rng.integers(0, 256, n, dtype=np.uint8)


def attn_case(name, seed, *, B, next_n, Hq, Hkv, D, bs, lens, kv_kind, scale_mode,
              q_dist="normal", causal=True, num_blocks=None, max_blocks=None,
              max_context_len=None, zero_k_channel_frac=0.0, k_scale_range=(1e-2, 1e3),
              v_scale_range=(1e-2, 1e3), pt_scale_range=(0.01, 2.0), poison=True) -> AttnCase:
    """Build one paged-attention input.

    Physical ids are a random permutation of 1..num_blocks-1 handed out in
    logical order; block 0 is the null block. Unused pages hold random bytes.
    The null block and the tail slots past each sequence's length hold NaN
    bytes (poison=True), so a kernel that reads them shows it. INT codes are
    uniform; a per-tensor INT scale is uniform in pt_scale_range (per-channel
    ones log-uniform in k_scale_range / v_scale_range).
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    assert lens.shape == (B,)
    pages = [(int(L) + bs - 1) // bs for L in lens]
    total = sum(pages)
    if num_blocks is None:
        num_blocks = int(total * 1.25) + 1
    assert num_blocks >= total + 1
    max_ctx = int(max_context_len if max_context_len is not None else max(1, int(lens.max())))
    if max_blocks is None:
        max_blocks = max(1, (max_ctx + bs - 1) // bs)
    rb = row_bytes(kv_kind, D)

    perm = rng.permutation(np.arange(1, num_blocks, dtype=np.int64))
    block_table = np.zeros((B, max_blocks), np.int32)
    cursor = 0
    for b in range(B):
        block_table[b, :pages[b]] = perm[cursor:cursor + pages[b]]
        cursor += pages[b]
    real = perm[:total]  # physical ids holding real pages, in (b, logical) order

    k_cache = rng.integers(0, 256, (num_blocks, bs, Hkv, rb), dtype=np.uint8)
    v_cache = rng.integers(0, 256, (num_blocks, bs, Hkv, rb), dtype=np.uint8)

    # token validity per real page slot
    valid = np.zeros((total, bs), bool)
    cursor = 0
    for b in range(B):
        for p in range(pages[b]):
            valid[cursor, :] = (p * bs + np.arange(bs)) < lens[b]
            cursor += 1

    shape_real = (total, bs, Hkv, D)
    k_scale = v_scale = None
    if kv_kind in (KV_F16, KV_BF16):
        assert scale_mode == SCALE_NONE
        kx = rng.standard_normal(shape_real, dtype=np.float32)
        vx = rng.standard_normal(shape_real, dtype=np.float32)
        if kv_kind == KV_F16:
            kc = kx.astype(np.float16).view(np.uint8).reshape(total, bs, Hkv, rb)
            vc = vx.astype(np.float16).view(np.uint8).reshape(total, bs, Hkv, rb)
        else:
            import torch
            kc = torch.from_numpy(kx).to(torch.bfloat16).view(torch.uint8).numpy().reshape(
                total, bs, Hkv, rb)
            vc = torch.from_numpy(vx).to(torch.bfloat16).view(torch.uint8).numpy().reshape(
                total, bs, Hkv, rb)
    elif kv_kind == KV_E4M3:
        assert scale_mode == SCALE_PER_TENSOR
        kx = rng.standard_normal(shape_real, dtype=np.float32)
        vx = rng.standard_normal(shape_real, dtype=np.float32)
        vmask = valid[:, :, None, None]
        # a cache with no real page (every length 0) takes scale 1
        kmax = np.abs(np.where(vmask, kx, 0)).max(initial=0.0)
        vmax = np.abs(np.where(vmask, vx, 0)).max(initial=0.0)
        k_scale = np.array([kmax / np.float32(448) if kmax > 0 else 1.0], np.float32)
        v_scale = np.array([vmax / np.float32(448) if vmax > 0 else 1.0], np.float32)
        kc = e4m3_codes_torch(kx / k_scale[0])
        vc = e4m3_codes_torch(vx / v_scale[0])
    else:
        lim = 127 if kv_kind == KV_INT8 else 7
        kcodes = rng.integers(-lim, lim + 1, shape_real).astype(np.int8)
        vcodes = rng.integers(-lim, lim + 1, shape_real).astype(np.int8)
        if zero_k_channel_frac > 0:
            nch = Hkv * D
            nzero = int(round(zero_k_channel_frac * nch))
            zch = rng.choice(nch, nzero, replace=False)
            kcodes.reshape(total, bs, nch)[:, :, zch] = 0
        if scale_mode == SCALE_PER_CHANNEL:
            lo, hi = k_scale_range
            k_scale = np.exp(rng.uniform(math.log(lo), math.log(hi), (Hkv, D))).astype(np.float32)
            lo, hi = v_scale_range
            v_scale = np.exp(rng.uniform(math.log(lo), math.log(hi), (Hkv, D))).astype(np.float32)
        elif scale_mode == SCALE_PER_TENSOR:
            k_scale = np.array([rng.uniform(*pt_scale_range)], np.float32)
            v_scale = np.array([rng.uniform(*pt_scale_range)], np.float32)
        if kv_kind == KV_INT8:
            kc = kcodes.view(np.uint8)
            vc = vcodes.view(np.uint8)
        else:
            def pack(c):
                u = (c.astype(np.int16) & 15).astype(np.uint8)
                return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
            kc, vc = pack(kcodes), pack(vcodes)

    if poison:
        # tail slots of real pages
        tail = ~valid
        if tail.any():
            n = int(tail.sum()) * Hkv * rb
            pk = _poison_byte_pattern(kv_kind, n, rng).reshape(-1, Hkv, rb)
            kc = kc.copy()
            vc = vc.copy()
            kc[tail] = pk
            vc[tail] = pk
    k_cache[real] = kc
    v_cache[real] = vc
    if poison:
        npb = bs * Hkv * rb
        k_cache[0] = _poison_byte_pattern(kv_kind, npb, rng).reshape(bs, Hkv, rb)
        v_cache[0] = _poison_byte_pattern(kv_kind, npb, rng).reshape(bs, Hkv, rb)

    if q_dist == "normal":
        q = rng.standard_normal((B, next_n, Hq, D), dtype=np.float32).astype(np.float16)
    else:
        lo, hi = q_dist
        q = rng.uniform(lo, hi, (B, next_n, Hq, D)).astype(np.float16)

    return AttnCase(name=name, q=q, k_cache=k_cache, v_cache=v_cache, kv_kind=kv_kind,
                    k_scale=k_scale, v_scale=v_scale,
                    k_scale_mode=scale_mode if k_scale is not None else SCALE_NONE,
                    v_scale_mode=scale_mode if v_scale is not None else SCALE_NONE,
                    block_table=block_table, context_lens=lens.astype(np.int32),
                    max_context_len=max_ctx, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                    softmax_scale=float(np.float32(1.0 / math.sqrt(D))), causal=causal)


def relocate(case: AttnCase, seed: int) -> AttnCase:
    """Same logical content under a fresh random physical placement.

    Every real page moves to a new physical id drawn from a new permutation of
    1..num_blocks-1; the null block stays at 0 and keeps its bytes; every other
    page gets fresh random bytes.
    """
    rng = np.random.default_rng(seed)
    nb = case.num_blocks
    perm = rng.permutation(np.arange(1, nb, dtype=np.int64))
    bt = case.block_table
    used = bt[bt > 0]
    # bt > 0 entries are exactly the real pages (the table is padded with 0)
    remap = np.zeros(nb, np.int64)
    remap[used] = perm[:used.size]
    k_new = np.random.default_rng(seed + 1).integers(0, 256, case.k_cache.shape, dtype=np.uint8)
    v_new = np.random.default_rng(seed + 2).integers(0, 256, case.v_cache.shape, dtype=np.uint8)
    k_new[0] = case.k_cache[0]
    v_new[0] = case.v_cache[0]
    k_new[remap[used]] = case.k_cache[used]
    v_new[remap[used]] = case.v_cache[used]
    new_bt = np.where(bt > 0, remap[bt], 0).astype(np.int32)
    return dataclasses.replace(case, k_cache=k_new, v_cache=v_new, block_table=new_bt)


def unpaged(case: AttnCase) -> AttnCase:
    """Same logical content laid out contiguously: sequence b occupies physical
    blocks in logical order, starting after the null block."""
    B = case.batch
    bs = case.block_size
    bt = case.block_table
    pages = [(int(L) + bs - 1) // bs for L in case.context_lens]
    total = sum(pages)
    nb = total + 1
    shape = (nb,) + case.k_cache.shape[1:]
    k_new = np.zeros(shape, np.uint8)
    v_new = np.zeros(shape, np.uint8)
    k_new[0] = case.k_cache[0]
    v_new[0] = case.v_cache[0]
    new_bt = np.zeros_like(bt)
    cursor = 1
    for b in range(B):
        for p in range(pages[b]):
            k_new[cursor] = case.k_cache[bt[b, p]]
            v_new[cursor] = case.v_cache[bt[b, p]]
            new_bt[b, p] = cursor
            cursor += 1
    return dataclasses.replace(case, k_cache=k_new, v_cache=v_new, block_table=new_bt)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def tiny_f16(seed=SEED_BASE + 0, poison=True) -> AttnCase:
    """fp16 KV, no quantization: B 2, GQA 4 (4 q heads / 1 KV head), D 64,
    block 16, lens {37, 70}, 16 blocks with block 0 as null block."""
    return attn_case("tiny_f16", seed, B=2, next_n=1, Hq=4, Hkv=1, D=64, bs=16, lens=[37, 70],
                     kv_kind=KV_F16, scale_mode=SCALE_NONE, num_blocks=16, poison=poison)


def fp8_decode(seed=SEED_BASE + 1, B=64, lo=512, hi=4096) -> AttnCase:
    """E4M3 per-tensor decode: B 64, 32 q / 8 KV heads, D 128, block 16,
    lens uniform in [512, 4096]."""
    rng = np.random.default_rng(seed + 10_000)
    lens = rng.integers(lo, hi + 1, B)
    return attn_case("fp8_decode", seed, B=B, next_n=1, Hq=32, Hkv=8, D=128, bs=16, lens=lens,
                     kv_kind=KV_E4M3, scale_mode=SCALE_PER_TENSOR, max_context_len=hi)


def int_perchan(kind=KV_INT8, seed=SEED_BASE + 2, B=32, L=8192) -> AttnCase:
    """INT8 / INT4 per-channel K and V scales: B 32, 16 q / 2 KV heads, D 256,
    block 32, len 8192, q uniform in [-100, 100], 10% of K channels all-zero.
    K scales log-uniform in [1e-2, 1e3]; V scales the same for INT4 and
    [1e-2, 65504/127] for INT8 so that dequantized V and outputs stay finite
    in fp16."""
    vr = (1e-2, 1e3) if kind == KV_INT4 else (1e-2, 65504.0 / 127.0)
    return attn_case("int4_perchan" if kind == KV_INT4 else "int8_perchan", seed, B=B, next_n=1,
                     Hq=16, Hkv=2, D=256, bs=32, lens=[L] * B, kv_kind=kind,
                     scale_mode=SCALE_PER_CHANNEL, q_dist=(-100.0, 100.0),
                     zero_k_channel_frac=0.10, k_scale_range=(1e-2, 1e3), v_scale_range=vr)


def fp8_verify(seed=SEED_BASE + 3, B=16, lo=4096, hi=16384) -> AttnCase:
    """E4M3 multi-row verify: B 16, next_n 4 causal, 64 q / 8 KV heads, D 128,
    block 32, lens uniform in [4096, 16384]."""
    rng = np.random.default_rng(seed + 10_000)
    lens = rng.integers(lo, hi + 1, B)
    return attn_case("fp8_verify", seed, B=B, next_n=4, Hq=64, Hkv=8, D=128, bs=32, lens=lens,
                     kv_kind=KV_E4M3, scale_mode=SCALE_PER_TENSOR, causal=True,
                     max_context_len=hi)


def fp8_prefill(seed=SEED_BASE + 7, B=8, next_n=256, lo=4096, hi=16384) -> AttnCase:
    """E4M3 chunked prefill: B 8, next_n 256 causal, 64 q / 8 KV heads, D 128,
    block 32, lens uniform in [4096, 16384] (the chunk's 256 tokens included)."""
    rng = np.random.default_rng(seed + 10_000)
    lens = rng.integers(lo, hi + 1, B)
    return attn_case("fp8_prefill", seed, B=B, next_n=next_n, Hq=64, Hkv=8, D=128, bs=32,
                     lens=lens, kv_kind=KV_E4M3, scale_mode=SCALE_PER_TENSOR, causal=True,
                     max_context_len=hi)


# ---------------------------------------------------------------------------
# MXFP4 paged MQA logits
# ---------------------------------------------------------------------------

# probabilities of the E2M1 magnitude codes 0..7 (values 0, .5, 1, 1.5, 2, 3, 4, 6):
# a bell shape, roughly what normally distributed values quantized per 32 look like
_E2M1_MAG_P = np.array([0.10, 0.16, 0.16, 0.14, 0.12, 0.14, 0.10, 0.08])


def _e2m1_nibbles(rng, shape):
    mag = rng.choice(8, size=shape, p=_E2M1_MAG_P).astype(np.uint8)
    sign = rng.integers(0, 2, shape, dtype=np.uint8) << 3
    return mag | sign


@dataclasses.dataclass
class LogitsCase:
    name: str
    q: np.ndarray  # uint8 [B, next_n, H, D/2]
    sf_q: np.ndarray  # int32 [B, next_n, H]
    kv_fused: np.ndarray  # uint8 [num_blocks, bs, 1, D/2 + D/32]
    weights: np.ndarray  # float32 [B*next_n, H]
    context_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks]
    max_context_len: int
    sf_vec_size: int = 32

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def next_n(self):
        return self.q.shape[1]

    @property
    def num_heads(self):
        return self.q.shape[2]

    @property
    def head_dim(self):
        return self.q.shape[3] * 2

    @property
    def block_size(self):
        return self.kv_fused.shape[1]

    def kv_bytes_visible(self) -> int:
        D = self.head_dim
        return int(self.context_lens.astype(np.int64).sum()) * (D // 2 + D // self.sf_vec_size)


def logits_case(name, seed, *, B, next_n, H, D, bs, lens, max_context_len, sf_lo=125, sf_hi=129,
                num_blocks=None, table_cols=None, poison=True) -> LogitsCase:
    """One MXFP4 paged MQA logits input. Codes and UE8M0 exponents are drawn
    directly; exponents in [sf_lo, sf_hi] keep the spread of (sf_q + sf_k)
    over a head's four 32-groups at most 2*(sf_hi - sf_lo)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    sf_vec = 32
    pages = [(int(L) + bs - 1) // bs for L in lens]
    total = sum(pages)
    if num_blocks is None:
        num_blocks = int(total * 1.25) + 1
    if table_cols is None:
        table_cols = max(1, ((max_context_len + 127) // 128 * 128) // bs)
    perm = rng.permutation(np.arange(1, num_blocks, dtype=np.int64))
    bt = np.zeros((B, table_cols), np.int32)
    cursor = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[cursor:cursor + pages[b]]
        cursor += pages[b]
    real = perm[:total]

    data_bytes = bs * D // 2
    sf_bytes = bs * D // sf_vec
    blk_bytes = data_bytes + sf_bytes
    kv = rng.integers(0, 256, (num_blocks, blk_bytes), dtype=np.uint8)
    nib = _e2m1_nibbles(rng, (total, bs, D))
    kv_data = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8).reshape(total, data_bytes)
    kv_sf = rng.integers(sf_lo, sf_hi + 1, (total, bs, D // sf_vec), dtype=np.uint8)
    if poison:
        cursor = 0
        for b in range(B):
            for p in range(pages[b]):
                tail = (p * bs + np.arange(bs)) >= lens[b]
                kv_sf[cursor, tail] = 0xFF
                cursor += 1
    kv[real, :data_bytes] = kv_data
    kv[real, data_bytes:] = kv_sf.reshape(total, sf_bytes)
    if poison:
        kv[0, data_bytes:] = 0xFF
    kv_fused = kv.reshape(num_blocks, bs, 1, D // 2 + D // sf_vec)

    qn = _e2m1_nibbles(rng, (B, next_n, H, D))
    q = (qn[..., 0::2] | (qn[..., 1::2] << 4)).astype(np.uint8)
    sfb = rng.integers(sf_lo, sf_hi + 1, (B, next_n, H, 4), dtype=np.uint8)
    sf_q = sfb.view(np.int32).reshape(B, next_n, H).copy()  # byte g = bits 8g..8g+7 (little end.)
    weights = rng.standard_normal((B * next_n, H), dtype=np.float32)
    return LogitsCase(name=name, q=q, sf_q=sf_q, kv_fused=kv_fused, weights=weights,
                      context_lens=lens.astype(np.int32), block_table=bt,
                      max_context_len=int(max_context_len))


def mxfp4_logits(seed=SEED_BASE + 4, B=32, max_len=32768) -> LogitsCase:
    """MXFP4 paged MQA logits: B 32, next_n 2, 64 heads, D 128, block 64,
    lens uniform in [1, 32768], max_context_len 32768, table padded with 0 to
    round_up(len, 128) / 64 columns."""
    rng = np.random.default_rng(seed + 10_000)
    lens = rng.integers(1, max_len + 1, B)
    return logits_case("mxfp4_logits", seed, B=B, next_n=2, H=64, D=128, bs=64, lens=lens,
                       max_context_len=max_len)


# ---------------------------------------------------------------------------
# KV insert
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class InsertCase:
    k: np.ndarray  # float16 [T, Hkv, D], or uint16 bf16 bits when in_bf16
    v: np.ndarray
    slot_mapping: np.ndarray  # int64 [num_slots]
    num_blocks: int
    block_size: int
    kv_kind: int
    k_scale: np.ndarray | None
    v_scale: np.ndarray | None
    scale_mode: int
    k_cache: np.ndarray  # prefilled destination, uint8 [num_blocks, bs, Hkv, row_bytes]
    v_cache: np.ndarray
    in_bf16: bool = False

    def values(self, x):
        """float32 values of k or v."""
        if self.in_bf16:
            return (x.astype(np.uint32) << 16).view(np.float32)
        return x.astype(np.float32)


def insert_case(seed, *, T, Hkv, D, bs, kv_kind, scale_mode, slotless_tail=0, neg_slots=0,
                value_scale=1.0, in_dtype="f16", oob_slots=0) -> InsertCase:
    """New tokens k, v [T, Hkv, D] ~ N(0, value_scale^2) as fp16 (or bf16
    bits with in_dtype="bf16"), distinct random slots in blocks 1.., the last
    `slotless_tail` rows without a slot (num_slots = T - slotless_tail),
    `neg_slots` rows with slot -1 and `oob_slots` rows whose slot lies past the
    cache. The destination caches are prefilled with NaN bytes (0xFF)."""
    rng = np.random.default_rng(seed)
    num_slots = T - slotless_tail
    nb = (T + bs - 1) // bs + 3
    slots = rng.choice(np.arange(bs, nb * bs), num_slots, replace=False).astype(np.int64)
    if neg_slots:
        slots[rng.choice(num_slots, neg_slots, replace=False)] = -1
    if oob_slots:
        pick = rng.choice(np.flatnonzero(slots >= 0), oob_slots, replace=False)
        slots[pick] = nb * bs + rng.integers(0, 5 * bs, oob_slots)
    kx = rng.standard_normal((T, Hkv, D), dtype=np.float32) * value_scale
    vx = rng.standard_normal((T, Hkv, D), dtype=np.float32) * value_scale
    if in_dtype == "bf16":
        import torch
        k = torch.from_numpy(kx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        v = torch.from_numpy(vx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        k, v = kx.astype(np.float16), vx.astype(np.float16)
    k_scale = v_scale = None
    kf = (k.astype(np.uint32) << 16).view(np.float32) if in_dtype == "bf16" else k.astype(np.float32)
    vf = (v.astype(np.uint32) << 16).view(np.float32) if in_dtype == "bf16" else v.astype(np.float32)
    if scale_mode == SCALE_PER_TENSOR:
        lim = {KV_E4M3: 448.0, KV_INT8: 127.0, KV_INT4: 7.0}[kv_kind]
        k_scale = np.array([np.abs(kf).max() / lim], np.float32)
        v_scale = np.array([np.abs(vf).max() / lim], np.float32)
    elif scale_mode == SCALE_PER_CHANNEL:
        k_scale = np.exp(rng.uniform(-3, 1, (Hkv, D))).astype(np.float32)
        v_scale = np.exp(rng.uniform(-3, 1, (Hkv, D))).astype(np.float32)
    rb = row_bytes(kv_kind, D)
    kc = np.full((nb, bs, Hkv, rb), 0xFF, np.uint8)
    vc = np.full((nb, bs, Hkv, rb), 0xFF, np.uint8)
    return InsertCase(k=k, v=v, slot_mapping=slots, num_blocks=nb, block_size=bs,
                      kv_kind=kv_kind, k_scale=k_scale, v_scale=v_scale, scale_mode=scale_mode,
                      k_cache=kc, v_cache=vc, in_bf16=in_dtype == "bf16")


@dataclasses.dataclass
class Mxfp4InsertCase:
    k_bits: np.ndarray         # [T, D] uint16 bits of fp16 or bf16 values
    in_dtype: str              # "f16" or "bf16"
    slot_mapping: np.ndarray   # [num_slots] int64 (num_slots <= T; -1 = no slot)
    kv_fused: np.ndarray       # [num_blocks, bs, 1, D/2 + D/32] uint8, prefilled with 0xFF
    sf_interleaved: bool


def mxfp4_insert_case(seed, *, T, D=128, bs=64, in_dtype="f16", slotless_tail=0, neg_slots=0,
                      sf_interleaved=False, spread=8.0) -> Mxfp4InsertCase:
    """New key rows [T, D]: N(0, 1) values times a per-row factor 2^u, u uniform
    in [-spread, spread], as fp16 or bf16 bits; a few exact zeros and one
    all-zero row. Distinct random slots in blocks 1..; the last `slotless_tail`
    rows have no slot and `neg_slots` rows have slot -1. The destination is
    prefilled with 0xFF so untouched bytes are visible."""
    import torch
    rng = np.random.default_rng(seed)
    num_slots = T - slotless_tail
    nb = (T + bs - 1) // bs + 3
    slots = rng.choice(np.arange(bs, nb * bs), num_slots, replace=False).astype(np.int64)
    if neg_slots:
        slots[rng.choice(num_slots, neg_slots, replace=False)] = -1
    x = rng.standard_normal((T, D)).astype(np.float32)
    x *= np.exp2(rng.uniform(-spread, spread, (T, 1))).astype(np.float32)
    x[rng.random((T, D)) < 0.02] = 0.0
    x[0] = 0.0
    t = torch.from_numpy(x).to(torch.bfloat16 if in_dtype == "bf16" else torch.float16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    kv = np.full((nb, bs, 1, D // 2 + D // 32), 0xFF, np.uint8)
    return Mxfp4InsertCase(k_bits=bits, in_dtype=in_dtype, slot_mapping=slots, kv_fused=kv,
                           sf_interleaved=sf_interleaved)


def with_selection(case: AttnCase, seed: int, topk: int, window: int = 128,
                   junk: int = 4) -> tuple:
    """A selection for every query row of `case`, as a top-k over indexer
    logits would give it: the last `window` tokens of the sequence plus random
    earlier ones, at most topk distinct ids per row in random order, padded
    with -1. `junk` extra entries per row repeat an id or fall outside [0, L)
    (they must select nothing more). Returns (case, sel int32 [B, next_n, topk + junk])."""
    rng = np.random.default_rng(seed)
    B, N = case.batch, case.next_n
    sel = np.full((B, N, topk + junk), -1, np.int32)
    for b in range(B):
        L = int(case.context_lens[b])
        for i in range(N):
            if L == 0:
                continue
            recent = np.arange(max(0, L - window), L)
            k = min(topk, L)
            rest = np.setdiff1d(np.arange(L), recent)
            extra = rng.choice(rest, min(max(0, k - recent.size), rest.size), replace=False)
            ids = np.concatenate([recent[-k:], extra])[:k]
            rng.shuffle(ids)
            sel[b, i, :ids.size] = ids
            j = [ids[0] if ids.size else -1, L, L + 17, -5][:junk]
            sel[b, i, topk:topk + len(j)] = j
    return case, sel


def fp8_sparse_verify(seed=SEED_BASE + 6, topk=2048, window=512):
    """The E4M3 verify workload (B 16, next_n 4, 64 q / 8 KV heads, D 128,
    block 32, lens uniform in [4096, 16384]) with a token selection per query
    row: the last 512 tokens plus random earlier ones, 2048 distinct ids per
    row, 4 junk entries. Returns (case, sel)."""
    case = dataclasses.replace(fp8_verify(), name="fp8_sparse_verify")
    return with_selection(case, seed, topk, window=window)
