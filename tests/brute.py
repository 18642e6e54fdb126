"""Independent brute-force references used to pin the oracle on tiny inputs.

Decoding goes through library conversions (torch float8/bfloat16 views, numpy
float16/int8 views) and attention through torch's scaled_dot_product_attention
in float64 on the CPU, so nothing here shares code with oracle/oracle.c.
"""
import numpy as np
import torch

import workloads as W


def decode_cache(cache: np.ndarray, kind: int, D: int) -> np.ndarray:
    """[nb, bs, Hkv, row_bytes] codes -> float32 [nb, bs, Hkv, D] code values."""
    c = np.ascontiguousarray(cache)
    if kind == W.KV_F16:
        return c.view(np.float16).astype(np.float32)
    if kind == W.KV_BF16:
        return torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).float().numpy()
    if kind == W.KV_E4M3:
        return torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    if kind == W.KV_INT8:
        return c.view(np.int8).astype(np.float32)
    lo = (c & 15).astype(np.uint8)
    hi = (c >> 4).astype(np.uint8)
    nib = np.stack([lo, hi], axis=-1).reshape(c.shape[:-1] + (D,))
    return ((nib << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.float32)


def dequant_cache(cache, kind, D, scale, mode):
    vals = decode_cache(cache, kind, D)
    if mode == W.SCALE_PER_TENSOR:
        vals = vals * np.float32(scale[0])
    elif mode == W.SCALE_PER_CHANNEL:
        vals = vals * scale.astype(np.float32)[None, None, :, :]
    return vals.astype(np.float32)


def gather(vals, block_table_row, L, bs):
    t = np.arange(L)
    return vals[block_table_row[t // bs], t % bs]  # [L, Hkv, D]


def attention_sdpa(case: W.AttnCase) -> np.ndarray:
    """float64 [B, next_n, Hq, D] via torch SDPA on gathered, dequantized K/V."""
    D = case.head_dim
    K = dequant_cache(case.k_cache, case.kv_kind, D, case.k_scale, case.k_scale_mode)
    V = dequant_cache(case.v_cache, case.kv_kind, D, case.v_scale, case.v_scale_mode)
    B, N, Hq, _ = case.q.shape
    group = Hq // case.num_kv_heads
    out = np.zeros((B, N, Hq, D), np.float64)
    for b in range(B):
        L = int(case.context_lens[b])
        if L == 0:
            continue
        kb = torch.from_numpy(gather(K, case.block_table[b], L, case.block_size).astype(np.float64))
        vb = torch.from_numpy(gather(V, case.block_table[b], L, case.block_size).astype(np.float64))
        kb = kb.permute(1, 0, 2).repeat_interleave(group, dim=0)[None]  # [1, Hq, L, D]
        vb = vb.permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
        qb = torch.from_numpy(case.q[b].astype(np.float64)).permute(1, 0, 2)[None]  # [1,Hq,N,D]
        t = np.arange(L)
        pos = L - N + np.arange(N)
        vis = (t[None, :] <= pos[:, None]) if case.causal else np.ones((N, L), bool)
        mask = torch.from_numpy(vis)
        o = torch.nn.functional.scaled_dot_product_attention(
            qb, kb, vb, attn_mask=mask, scale=float(case.softmax_scale))
        o = o[0].permute(1, 0, 2).numpy()  # [N, Hq, D]
        o[~vis.any(1)] = 0.0
        out[b] = o
    return out


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def logits_exact(case: W.LogitsCase) -> np.ndarray:
    """float64 per-head dot products S[r, t, h] (exact for the workload's
    exponent spread) via table lookup and ldexp."""
    B, N, H, Dh = case.q.shape
    D = Dh * 2
    bs = case.block_size
    qn = np.stack([case.q & 15, case.q >> 4], -1).reshape(B, N, H, D)
    qsf = case.sf_q.view(np.uint8).reshape(B, N, H, 4).astype(np.int64)
    qv = E2M1[qn] * np.ldexp(1.0, np.repeat(qsf, 32, axis=-1) - 127)
    kvb = case.kv_fused.reshape(case.kv_fused.shape[0], -1)
    data = kvb[:, : bs * D // 2].reshape(-1, bs, D // 2)
    sf = kvb[:, bs * D // 2:].reshape(-1, bs, D // 32).astype(np.int64)
    out = []
    for b in range(B):
        L = int(case.context_lens[b])
        t = np.arange(L)
        blk = case.block_table[b, t // bs]
        kd = data[blk, t % bs]
        kn = np.stack([kd & 15, kd >> 4], -1).reshape(L, D)
        ks = sf[blk, t % bs]
        kv = E2M1[kn] * np.ldexp(1.0, np.repeat(ks, 32, axis=-1) - 127)
        out.append(np.einsum("nhd,td->nth", qv[b], kv))  # [N, L, H]
    return out
