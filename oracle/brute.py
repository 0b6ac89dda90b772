"""Brute-force dense check of the oracle -- TEST INFRASTRUCTURE ONLY.

An implementation independent of oracle.c, for tiny inputs: rows are
dequantised with PyTorch's own float8_e4m3fn and bfloat16 conversions (not the
oracle's decoder), logits come from one dense fp64 matrix product over the
gathered rows, and the softmax from scipy's logsumexp.  It follows the same
definition: attention of each head over the rows its top-k list selects, with
keys and values equal to the dequantised 512-wide latent row.
"""

from __future__ import annotations

import numpy as np
import torch
from scipy.special import logsumexp


def dequant_rows_torch(rows: np.ndarray, row_format: int = 0) -> np.ndarray:
    """rows uint8 [N,640] (format 0) or [N,584] (format 1, UE8M0 scales) ->
    K fp64 [N,512] using torch's dtype conversions; a UE8M0 byte e is the
    power of two 2^(e - 127) (torch.exp2 in fp64), 255 NaN."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    t = torch.from_numpy(rows)
    codes = t[:, :448].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    if row_format == 1:
        e = t[:, 448:455].to(torch.float64)                                     # [N,7]
        scales = torch.where(e == 255, torch.full_like(e, float("nan")), torch.exp2(e - 127))
        rope = t[:, 456:584].contiguous().view(torch.bfloat16).to(torch.float64)
    else:
        scales = t[:, 448:476].contiguous().view(torch.float32).to(torch.float64)  # [N,7]
        rope = t[:, 480:608].contiguous().view(torch.bfloat16).to(torch.float64)
    nope = codes * scales.repeat_interleave(64, dim=1)
    return torch.cat([nope, rope], dim=1).numpy().reshape(n, 512)


def q_values(q_bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(q_bits, dtype=np.uint16).view(np.int16)) \
        .view(torch.bfloat16).to(torch.float64).numpy()


def _attend(q_b, K, scale):
    z = scale * (q_b @ K.T)                    # [H,n]
    l = logsumexp(z, axis=1)
    p = np.exp(z - l[:, None])
    return p @ K, l


def brute_decode(q_bits, cache, kv_seq_stride, idx, seqlens, scale, row_format=0):
    """Dense fp64 attention restricted to the selected rows (tiny inputs)."""
    q = q_values(q_bits)                       # [B,H,512]
    B, H, _ = q.shape
    cache = cache.reshape(B, kv_seq_stride, 584 if row_format == 1 else 640)
    out = np.zeros((B, H, 512))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        sel = [int(t) for t in idx[b] if 0 <= t < seqlens[b]]
        if not sel:
            continue
        K = dequant_rows_torch(cache[b, sel], row_format)  # [n,512]
        out[b], lse[b] = _attend(q[b], K, scale)
    return out, lse


def brute_decode_paged(q_bits, pool, num_pages, page_size, block_table, idx, seqlens, scale,
                       row_format=0):
    """Dense fp64 attention over a paged pool (tiny inputs): the rows of the
    kept entries are found with one vectorised block-table lookup
    (page = table[b, t // page_size], row = page * page_size + t % page_size)."""
    q = q_values(q_bits)
    B, H, _ = q.shape
    rows = pool.reshape(num_pages * page_size, 584 if row_format == 1 else 640)
    idx = np.asarray(idx, dtype=np.int64)
    pps = block_table.shape[1]
    logical_page = np.where(idx >= 0, idx, 0) // page_size
    in_table = logical_page < pps
    page = np.take_along_axis(block_table.astype(np.int64), np.minimum(logical_page, pps - 1), axis=1)
    keep = (idx >= 0) & (idx < np.asarray(seqlens)[:, None]) & in_table & (page >= 0) & (page < num_pages)
    phys = page * page_size + np.where(idx >= 0, idx, 0) % page_size
    out = np.zeros((B, H, 512))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        if not keep[b].any():
            continue
        K = dequant_rows_torch(rows[phys[b][keep[b]]], row_format)
        out[b], lse[b] = _attend(q[b], K, scale)
    return out, lse
