"""Exact attention forward, by definition, in float64 (test infrastructure).

Follows "Flash Attention 3：让 GPU 跑满的注意力计算", §1.2 (standard
attention: S = Q K^T, P = softmax(S), O = P V, with S materialised) and §2.2
(softmax(x)_i = e^{x_i} / sum_j e^{x_j}).  The softmax scale multiplies S
(the blog's varlen call passes ``softmax_scale = 1/sqrt(d_k)``, §5.2).

Readings where the pages are silent:

* causal = keep key j for query i iff j <= i, aligned at row 0 (top-left),
  for any Nq, Nk; per sequence with local indices in varlen mode;
* lse_i = logsumexp_j S_ij (natural log, scaled scores, unmasked keys);
* a row with no unmasked key (only when Nk = 0) gives O_i = 0, lse_i = -inf.

Only a numpy matmul is used as a library primitive; there is no blocking.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: take its exact values
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def causal_mask(nq: int, nk: int) -> np.ndarray:
    """Boolean [nq, nk], True where key j is visible to query i (j <= i)."""
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return j <= i


def scores(q, k, scale: float, causal: bool = False) -> np.ndarray:
    """S = scale * Q K^T over the last two axes; masked entries are -inf."""
    q = _f64(q)
    k = _f64(k)
    s = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    if causal:
        s = np.where(causal_mask(q.shape[-2], k.shape[-2]), s, -np.inf)
    return s


def softmax_rows(s: np.ndarray):
    """Row softmax of a score matrix with -inf for masked entries.

    Returns ``(P, m, l)`` with m the row max, l = sum_j exp(S_ij - m) and
    P = exp(S - m) / l.  A row whose entries are all -inf (or which has no
    entries) gets P = 0, m = -inf, l = 0.
    """
    s = np.asarray(s, dtype=np.float64)
    if s.shape[-1] == 0:
        m = np.full(s.shape[:-1], -np.inf)
    else:
        m = s.max(axis=-1)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[..., None])  # exp(-inf) = 0 exactly for masked entries
    e = np.where(live[..., None], e, 0.0)
    l = e.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(live[..., None], e / np.where(live, l, 1.0)[..., None], 0.0)
    return p, m, l


def attention(q, k, v, scale: float, causal: bool = False):
    """O = softmax(scale Q K^T [+causal]) V and lse, over the last two axes.

    q: [..., Nq, d]; k, v: [..., Nk, d] (any leading batch/head axes).
    Returns float64 ``(O [..., Nq, d], lse [..., Nq])``.
    """
    v = _f64(v)
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    o = np.matmul(p, v)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False):
    """Variable-length batch: q [H, Tq, d], k/v [H, Tk, d] packed along tokens.

    Sequence b owns rows [cu_q[b], cu_q[b+1]) of q and [cu_k[b], cu_k[b+1])
    of k and v ("Flash Attention 3：让 GPU 跑满的注意力计算", §5.2: cumulative
    lengths [0, len1, len1+len2, ...]).  Each sequence is an independent
    attention problem; causal uses indices local to the sequence.
    Returns ``(O [H, Tq, d], lse [H, Tq])``.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    H, Tq, d = q.shape
    o = np.zeros((H, Tq, v.shape[-1]))
    lse = np.full((H, Tq), -np.inf)
    for b in range(len(cu_q) - 1):
        qs = slice(cu_q[b], cu_q[b + 1])
        ks = slice(cu_k[b], cu_k[b + 1])
        ob, lb = attention(q[:, qs], k[:, ks], v[:, ks], scale, causal)
        o[:, qs] = ob
        lse[:, qs] = lb
    return o, lse


def attention_rows(q, k, v, rows, scale: float, causal: bool = False):
    """O and lse for selected query rows of one head (q [Nq, d], k/v [Nk, d]).

    Used to check sampled outputs of problems too large to materialise
    whole.  ``rows`` are query indices; causal keeps keys j <= row.
    """
    q = _f64(q)[np.asarray(rows)]
    k = _f64(k)
    v = _f64(v)
    s = float(scale) * (q @ k.T)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j <= np.asarray(rows)[:, None], s, -np.inf)
    p, m, l = softmax_rows(s)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse
