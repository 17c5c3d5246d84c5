"""Tiled attention with the online-softmax recurrence, float64 (test infrastructure).

Follows "Flash Attention 3：让 GPU 跑满的注意力计算":

* §2.1 block tiling: Q in blocks of Br rows, K and V in blocks of Bc rows;
  the outer loop runs over the K/V blocks j, the inner loop over the Q
  blocks i; S_ij = Q_i K_j^T and softmax(S_ij) V_j are formed per block and
  only the final O_i is kept;
* §2.2 the update equations for block j with running statistics m, l:
  m_new = max(m_old, m_j);
  l_new = l_old e^{m_old - m_new} + l_j e^{m_j - m_new};
  O_new = O_old l_old e^{m_old - m_new} / l_new + P_j V_j e^{m_j - m_new} / l_new.

Reading (the blog leaves P_j, m_j, l_j undefined): m_j is the row max of the
block's scores, P_j = exp(S_j - m_j) and l_j = rowsum P_j; this is the only
reading under which the blog's claim that tiled and one-shot softmax agree
holds.  The second form, ``form="deferred"``, keeps O unnormalised,
rescales it by e^{m_old - m_new} and divides by l once at the end (the
"fewer non-matmul operations" reordering of §3.1); it is algebraically the
same.

Masked entries are -inf.  A row that has seen only masked entries keeps
(m, l, O) = (-inf, 0, 0): factors e^{-inf - m} are taken as exactly 0 and
nothing is divided by l = 0.
"""

from __future__ import annotations

import numpy as np

from .exact import _f64, causal_mask


def _exp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """e^{a-b}, taken as exactly 0 when a or b is -inf."""
    a, b = np.broadcast_arrays(np.asarray(a, np.float64), np.asarray(b, np.float64))
    out = np.zeros(a.shape)
    ok = np.isfinite(a) & np.isfinite(b)
    out[ok] = np.exp(a[ok] - b[ok])
    return out


def attention_tiled(q, k, v, scale: float, causal: bool = False,
                    br: int = 64, bc: int = 64, form: str = "normalized"):
    """One head: q [Nq, d], k/v [Nk, d].  Returns float64 (O [Nq, d], lse [Nq])."""
    if form not in ("normalized", "deferred"):
        raise ValueError(form)
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    nq, nk = q.shape[0], k.shape[0]
    dv = v.shape[1]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    o = np.zeros((nq, dv))
    vis = causal_mask(nq, nk) if causal else None

    for j0 in range(0, nk, bc):  # outer loop: K/V blocks
        kj, vj = k[j0:j0 + bc], v[j0:j0 + bc]
        for i0 in range(0, nq, br):  # inner loop: Q blocks
            rows = slice(i0, i0 + br)
            s = float(scale) * (q[rows] @ kj.T)
            if causal:
                s = np.where(vis[rows, j0:j0 + bc], s, -np.inf)
            m_j = s.max(axis=1)
            p_j = np.exp(s - np.where(np.isfinite(m_j), m_j, 0.0)[:, None])
            p_j[~np.isfinite(m_j)] = 0.0
            l_j = p_j.sum(axis=1)

            m_old, l_old, o_old = m[rows], l[rows], o[rows]
            m_new = np.maximum(m_old, m_j)
            a_old = _exp_diff(m_old, m_new)  # e^{m_old - m_new}
            a_j = _exp_diff(m_j, m_new)  # e^{m_j - m_new}
            l_new = l_old * a_old + l_j * a_j
            pv = p_j @ vj
            if form == "normalized":
                live = l_new > 0
                den = np.where(live, l_new, 1.0)[:, None]
                o_new = np.where(live[:, None],
                                 o_old * (l_old * a_old)[:, None] / den + pv * a_j[:, None] / den,
                                 0.0)
            else:
                o_new = o_old * a_old[:, None] + pv * a_j[:, None]
            m[rows], l[rows], o[rows] = m_new, l_new, o_new

    if form == "deferred":
        live = l > 0
        o = np.where(live[:, None], o / np.where(live, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse
