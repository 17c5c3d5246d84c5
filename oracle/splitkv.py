"""Attention split over key chunks, and the merge of the partial results, in
float64 (test infrastructure).

"Flash Attention 3：让 GPU 跑满的注意力计算", §2.2 combines the softmax of two
disjoint key blocks through their row maxima m and sums l:
m = max(m1, m2), l = e^{m1 - m} l1 + e^{m2 - m} l2, and the normalised
outputs weighted by e^{m_s - m} l_s / l.  Written with lse_s = m_s + ln l_s
this is, for any number of chunks,

    lse = ln sum_s e^{lse_s},    O = sum_s e^{lse_s - lse} O_s,

which is why the forward pass exports lse.  The "FlashAttention-3" wiki page
lists FlashDecoding (attention split along the keys, then merged) among the
related techniques.

Readings where the pages are silent:

* the keys are cut into ``num_splits`` chunks of ceil(Nk / num_splits) rows,
  in order (the last chunks may be short or empty);
* causal masking uses absolute key indices (top-left: key j visible to query
  i iff j <= i), whatever chunk the key falls in;
* a chunk with no visible key contributes O_s = 0, lse_s = -inf and weight 0;
  a row with no visible key at all gives O = 0, lse = -inf.

Only numpy matmul/exp/log are used; the merge is computed with the largest
lse_s subtracted first so that no exponential overflows.
"""

from __future__ import annotations

import numpy as np

from .exact import _f64, softmax_rows


def split_bounds(nk: int, num_splits: int):
    """Key ranges [begin, end) of the chunks, chunk length ceil(nk / num_splits)."""
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    n = -(-nk // num_splits) if nk > 0 else 0
    return [(min(s * n, nk), min((s + 1) * n, nk)) for s in range(num_splits)]


def attention_partial(q, k, v, scale: float, causal: bool, k_begin: int, k_end: int):
    """Normalised attention of the queries over keys [k_begin, k_end) only.

    q: [..., Nq, d]; k, v: [..., Nk, d] (whole key tensors; the chunk is sliced
    here so that causal masking sees absolute key indices).
    Returns ``(O_s [..., Nq, d], lse_s [..., Nq])``.
    """
    q = _f64(q)
    k = _f64(k)[..., k_begin:k_end, :]
    v = _f64(v)[..., k_begin:k_end, :]
    s = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    if causal:
        i = np.arange(q.shape[-2])[:, None]
        j = k_begin + np.arange(k.shape[-2])[None, :]
        s = np.where(j <= i, s, -np.inf)
    p, m, l = softmax_rows(s)
    o = np.matmul(p, v)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def merge(o_parts, lse_parts):
    """Combine partial results over disjoint key chunks.

    o_parts: [S, ..., Nq, d]; lse_parts: [S, ..., Nq].  Returns ``(O, lse)``
    with lse = ln sum_s e^{lse_s} and O = sum_s e^{lse_s - lse} O_s.
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    w = np.where(live[None], np.exp(lse_parts - m_safe[None]), 0.0)  # e^{lse_s - m}, 0 for empty chunks
    tot = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(live[..., None], (w[..., None] * o_parts).sum(axis=0) / np.where(live, tot, 1.0)[..., None], 0.0)
        lse = np.where(live, m_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    return o, lse


def attention_splitkv(q, k, v, scale: float, causal: bool, num_splits: int, parts: bool = False):
    """Attention computed chunk by chunk over the keys and merged.

    Returns ``(O, lse)``, or ``(O, lse, o_parts, lse_parts)`` with
    ``parts=True`` (o_parts [S, ..., Nq, d], lse_parts [S, ..., Nq]).
    """
    nk = _f64(k).shape[-2]
    outs = [attention_partial(q, k, v, scale, causal, b, e) for b, e in split_bounds(nk, num_splits)]
    o_parts = np.stack([o for o, _ in outs])
    lse_parts = np.stack([lse for _, lse in outs])
    o, lse = merge(o_parts, lse_parts)
    if parts:
        return o, lse, o_parts, lse_parts
    return o, lse
