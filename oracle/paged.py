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
"""

from __future__ import annotations

import numpy as np

from .exact import _f64, attention


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
