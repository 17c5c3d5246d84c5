"""Gradients of exact attention, by definition, in float64 (test infrastructure).

The pages measure a backward pass of the attention they compute
("FlashAttention-3" wiki page, the "Measured (H100 80GB SXM5)" table: the
speed-up over FlashAttention-2 backward) and name E5M2 as the fp8 format for
back-propagation ("Flash Attention 3：让 GPU 跑满的注意力计算", §4.1.2), but
print no algorithm for it.  The result is nevertheless fixed: it is the
derivative of the forward definition (§1.2 and §2.2 of that blog post, as in
``oracle.exact``)

    S = scale Q K^T [+ causal -inf],  P = softmax_rows(S),  O = P V

for a loss L with dL/dO = dO.  Written out by the chain rule:

    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - delta_i),   delta_i = sum_j P_ij dP_ij
    dQ = scale dS K,   dK = scale dS^T Q

(the softmax Jacobian of row i is diag(p) - p p^T; delta_i also equals
sum_c dO_ic O_ic, since dP_i . p = dO_i . (P V)_i).  Masked entries have
P = 0, hence dS = 0; a row with no visible key contributes nothing.

Only numpy matmuls are used; nothing is tiled or recomputed.
"""

from __future__ import annotations

import numpy as np

from .exact import _f64, scores, softmax_rows


def attention_backward(q, k, v, do, scale: float, causal: bool = False):
    """(dQ, dK, dV) of L = sum(dO * O) for O = softmax(scale Q K^T [+causal]) V.

    q, do: [..., Nq, d]; k, v: [..., Nk, d].  Returns float64 arrays of the
    shapes of q, k, v.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _, _ = softmax_rows(scores(q, k, scale, causal))
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    delta = (p * dp).sum(axis=-1)
    ds = p * (dp - delta[..., None])
    dq = float(scale) * np.matmul(ds, k)
    dk = float(scale) * np.matmul(np.swapaxes(ds, -1, -2), q)
    return dq, dk, dv


def row_delta(o, do):
    """delta_i = sum_c dO_ic O_ic: the row term of dS computed from the
    forward output (the quantity a recomputing backward reads instead of
    forming P dP^T)."""
    return (_f64(o) * _f64(do)).sum(axis=-1)


def intermediates(q, k, v, do, scale: float, causal: bool = False):
    """The matrices of ``attention_backward``: dict with P, dP, delta, dS (for
    error bounds in tests)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _, _ = softmax_rows(scores(q, k, scale, causal))
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    delta = (p * dp).sum(axis=-1)
    return {"P": p, "dP": dp, "delta": delta, "dS": p * (dp - delta[..., None])}


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, scale: float, causal: bool = False):
    """Gradients for a packed variable-length batch: q, do [H, Tq, d], k, v
    [H, Tk, d], sequence s owning rows cu_q[s]:cu_q[s+1] (queries) and
    cu_k[s]:cu_k[s+1] (keys); each sequence is an independent attention, so
    its gradients are ``attention_backward`` on its rows (zero elsewhere)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for s in range(len(cu_q) - 1):
        qa, qb, ka, kb = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        g = attention_backward(q[:, qa:qb], k[:, ka:kb], v[:, ka:kb], do[:, qa:qb], scale, causal)
        dq[:, qa:qb], dk[:, ka:kb], dv[:, ka:kb] = g
    return dq, dk, dv
