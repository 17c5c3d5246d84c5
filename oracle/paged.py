"""Attention over a paged key/value cache, by definition (test infrastructure).

"Flash Attention 3：让 GPU 跑满的注意力计算", §5.3 describes attention with a
paged KV cache (PagedAttention): the pages of each sequence are collected
from the page table into a contiguous buffer and ordinary attention runs on
it.  This module is that definition written out:

* the cache holds ``num_pages`` pages of ``page_size`` token rows, each row
  the keys (or values) of all H heads: ``[num_pages, page_size, H, d]``;
* ``block_table[b, j]`` is the page that holds tokens j*page_size ..
  (j+1)*page_size - 1 of sequence b; ``seqlens[b]`` tokens are valid;
* sequence b's keys for head h are the rows t = 0 .. seqlens[b]-1 of
  ``k_cache[block_table[b, t // page_size], t % page_size, h]``;
* every query of sequence b attends to all of them (no causal mask: the
  queries are the newest tokens, as in decoding), ``oracle.attention``.

A sequence with no valid token gives O = 0 and lse = -inf.

Low-precision caches (§4.1.3 of the same post: INT8 and FP8 KV caches) hold
8-bit codes and one fp32 scale per (token, head); the cached key is
scale * decode(code), with decode the e4m3 format definition (``oracle.fp8``)
or the signed 8-bit integer.  ``dequantize`` writes that out; attention then
runs on the dequantized cache.
"""

from __future__ import annotations

import numpy as np

from .exact import _f64, attention
from .fp8 import e4m3_decode


def gather(cache, block_table, seqlens, b: int) -> np.ndarray:
    """Contiguous [H, seqlens[b], d] rows of sequence b, collected page by page."""
    cache = _f64(cache)
    page_size = cache.shape[1]
    n = int(seqlens[b])
    if n == 0:
        return np.zeros((cache.shape[2], 0, cache.shape[3]))
    pages = [cache[int(block_table[b, j])] for j in range((n + page_size - 1) // page_size)]
    rows = np.concatenate(pages, axis=0)[:n]        # [n, H, d]
    return np.transpose(rows, (1, 0, 2))            # [H, n, d]


def attention_paged(q, k_cache, v_cache, block_table, seqlens, scale: float):
    """q [B, H, Nq, d] -> (O [B, H, Nq, d], lse [B, H, Nq]) in float64."""
    q = _f64(q)
    block_table = np.asarray(block_table)
    seqlens = np.asarray(seqlens)
    B = q.shape[0]
    o = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -np.inf)
    for b in range(B):
        k = gather(k_cache, block_table, seqlens, b)
        v = gather(v_cache, block_table, seqlens, b)
        o[b], lse[b] = attention(q[b], k, v, scale, False)
    return o, lse


def dequantize(codes, scales, kind: str) -> np.ndarray:
    """codes uint8 [num_pages, page_size, H, d], scales [num_pages, page_size, H]
    -> float64 cache scale * decode(code); kind "e4m3" or "int8"."""
    codes = np.asarray(codes, dtype=np.uint8)
    if kind == "e4m3":
        vals = e4m3_decode(codes)
    elif kind == "int8":
        vals = codes.view(np.int8).astype(np.float64)
    else:
        raise ValueError(kind)
    return np.asarray(scales, dtype=np.float64)[..., None] * vals


def attention_paged_quant(q, k_codes, v_codes, k_scales, v_scales, block_table, seqlens, scale: float, kind: str):
    """Attention over an 8-bit paged cache: the definition on the dequantized cache."""
    return attention_paged(q, dequantize(k_codes, k_scales, kind), dequantize(v_codes, v_scales, kind),
                           block_table, seqlens, scale)
