"""Pins of the attention-gradient oracle (CPU only).

``oracle.backward.attention_backward`` is held to things other than its own
formulas: central finite differences of L = sum(dO * O) through the forward
oracle (itself pinned in ``test_oracle_attention.py``), the calculus of a
two-key problem written out by hand, the one-key case (softmax constant),
symmetries of attention (a shift of every key leaves O unchanged, so the key
gradients sum to zero; Q -> tQ, K -> K/t leaves S unchanged, so
<dQ, Q> = <dK, K>), masking, and the identity delta_i = dO_i . O_i.
``test_mutations`` plants plausible mistakes into copies of the function and
checks that some pin catches each.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import backward as BW


def _problem(lead, nq, nk, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(lead + (nq, d)), rng.standard_normal(lead + (nk, d)),
            rng.standard_normal(lead + (nk, d)), rng.standard_normal(lead + (nq, d)))


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float((o * do).sum())


# ---------------------------------------------------------------- pin checks
# Each takes the gradient function under test (the oracle's, or a mutant).

def pin_finite_differences(grad):
    h = 1e-6
    for causal in (False, True):
        for nq, nk in ((5, 7), (6, 4), (4, 4)):
            q, k, v, do = _problem((2,), nq, nk, 3, seed=10 * nq + nk + causal)
            scale = 0.8
            got = grad(q, k, v, do, scale, causal)
            for which, x in enumerate((q, k, v)):
                num = np.zeros_like(x)
                for idx in np.ndindex(x.shape):
                    xp = x.copy()
                    xm = x.copy()
                    xp[idx] += h
                    xm[idx] -= h
                    args_p = [q, k, v]
                    args_m = [q, k, v]
                    args_p[which] = xp
                    args_m[which] = xm
                    num[idx] = (_loss(*args_p, do, scale, causal) - _loss(*args_m, do, scale, causal)) / (2 * h)
                np.testing.assert_allclose(got[which], num, rtol=0, atol=2e-7)


def pin_two_keys_closed_form(grad):
    # one query, two keys, d = 1: p = sigmoid(s_a - s_b), O = p v_a + (1-p) v_b
    qv, ka, kb, va, vb, g, scale = 0.9, 1.3, -0.4, 2.0, -1.5, 0.7, 0.6
    q = np.array([[qv]])
    k = np.array([[ka], [kb]])
    v = np.array([[va], [vb]])
    do = np.array([[g]])
    p = 1.0 / (1.0 + math.exp(-scale * qv * (ka - kb)))
    common = g * (va - vb) * p * (1 - p) * scale
    dq, dk, dv = grad(q, k, v, do, scale, False)
    np.testing.assert_allclose(dq[0, 0], common * (ka - kb), rtol=1e-13)
    np.testing.assert_allclose(dk[:, 0], [common * qv, -common * qv], rtol=1e-13)
    np.testing.assert_allclose(dv[:, 0], [g * p, g * (1 - p)], rtol=1e-13)


def pin_one_key(grad):
    q, k, v, do = _problem((3,), 6, 1, 4, seed=2)
    dq, dk, dv = grad(q, k, v, do, 0.5, False)
    assert np.all(np.abs(dq) <= 1e-15) and np.all(np.abs(dk) <= 1e-14)
    np.testing.assert_allclose(dv[:, 0, :], do.sum(axis=1), rtol=1e-14)


def pin_symmetries(grad):
    for causal in (False, True):
        q, k, v, do = _problem((2, 2), 9, 9, 5, seed=7 + causal)
        dq, dk, dv = grad(q, k, v, do, 0.4, causal)
        # shifting every key by one vector leaves each row of S shifted by a constant
        np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-12)
        # Q -> tQ, K -> K/t leaves S unchanged
        np.testing.assert_allclose((dq * q).sum(axis=(-1, -2)), (dk * k).sum(axis=(-1, -2)), rtol=1e-11)
        # O is linear in V, so dV is linear in dO
        rng = np.random.default_rng(1)
        do2 = rng.standard_normal(do.shape)
        dv2 = grad(q, k, v, do2, 0.4, causal)[2]
        dv12 = grad(q, k, v, do + 2.0 * do2, 0.4, causal)[2]
        np.testing.assert_allclose(dv12, dv + 2.0 * dv2, atol=1e-12)


def pin_masking(grad):
    q, k, v, do = _problem((), 4, 7, 3, seed=5)
    dq, dk, dv = grad(q, k, v, do, 0.7, True)
    assert np.all(dq[0] == 0.0)  # query 0 sees key 0 only: its softmax is constant
    assert np.all(dk[4:] == 0.0) and np.all(dv[4:] == 0.0)  # keys no query sees
    # key 3 is seen by query 3 only, through P_33
    p = oracle.softmax_rows(oracle.scores(q, k, 0.7, True))[0]
    np.testing.assert_allclose(dv[3], p[3, 3] * do[3], rtol=1e-13)


def pin_no_keys(grad):
    q, k, v, do = _problem((2,), 3, 0, 4, seed=1)
    dq, dk, dv = grad(q, k, v, do, 1.0, False)
    assert dq.shape == q.shape and np.all(dq == 0.0)
    assert dk.shape == k.shape and dv.shape == v.shape


def pin_repeated_pairs(grad):
    """Every (key, value) pair repeated m times, in any order: each copy takes
    1/m of the pair's softmax weight, so dQ is unchanged and each copy's dK
    and dV are the pair's over m.  The GPU test of key offsets beyond 2^31
    elements relies on it."""
    q, k, v, do = _problem((2,), 6, 5, 4, seed=11)
    m = 3
    perm = np.random.default_rng(2).permutation(5 * m)
    src = np.tile(np.arange(5), m)[perm]  # pair of each repeated key
    dq, dk, dv = grad(q, k, v, do, 0.8, False)
    dq_r, dk_r, dv_r = grad(q, k[:, src], v[:, src], do, 0.8, False)
    np.testing.assert_allclose(dq_r, dq, atol=1e-13)
    np.testing.assert_allclose(dk_r, dk[:, src] / m, atol=1e-13)
    np.testing.assert_allclose(dv_r, dv[:, src] / m, atol=1e-13)


PINS = [pin_finite_differences, pin_two_keys_closed_form, pin_one_key, pin_symmetries, pin_masking, pin_no_keys,
        pin_repeated_pairs]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(BW.attention_backward)


def test_row_delta_identity():
    """delta_i = sum_j P_ij dP_ij equals dO_i . O_i (what a recomputing
    backward reads from the forward output)."""
    for causal in (False, True):
        q, k, v, do = _problem((2,), 7, 5, 4, seed=3)
        o, _ = oracle.attention(q, k, v, 0.9, causal)
        it = BW.intermediates(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(BW.row_delta(o, do), it["delta"], atol=1e-13)
        dq, dk, dv = BW.attention_backward(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(dq, 0.9 * it["dS"] @ k, atol=1e-14)


# ---------------------------------------------------------------- mutations

def _parts(q, k, v, do, scale, causal):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    p = oracle.softmax_rows(oracle.scores(q, k, scale, causal))[0]
    dp = do @ np.swapaxes(v, -1, -2)
    return q, k, v, do, p, dp


def _no_delta(q, k, v, do, scale, causal):
    q, k, v, do, p, dp = _parts(q, k, v, do, scale, causal)
    ds = p * dp
    return scale * ds @ k, scale * np.swapaxes(ds, -1, -2) @ q, np.swapaxes(p, -1, -2) @ do


def _delta_unweighted(q, k, v, do, scale, causal):
    q, k, v, do, p, dp = _parts(q, k, v, do, scale, causal)
    ds = p * (dp - dp.sum(axis=-1, keepdims=True) / max(dp.shape[-1], 1))
    return scale * ds @ k, scale * np.swapaxes(ds, -1, -2) @ q, np.swapaxes(p, -1, -2) @ do


def _dk_no_scale(q, k, v, do, scale, causal):
    dq, dk, dv = BW.attention_backward(q, k, v, do, scale, causal)
    return dq, dk / scale, dv


def _dq_transposed(q, k, v, do, scale, causal):
    q, k, v, do, p, dp = _parts(q, k, v, do, scale, causal)
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dst = np.swapaxes(ds, -1, -2)
    return scale * dst @ k, scale * dst @ q, np.swapaxes(p, -1, -2) @ do


def _sign_flip(q, k, v, do, scale, causal):
    dq, dk, dv = BW.attention_backward(q, k, v, do, scale, causal)
    return -dq, -dk, dv


def _dv_unmasked(q, k, v, do, scale, causal):
    dq, dk, _ = BW.attention_backward(q, k, v, do, scale, causal)
    p = oracle.softmax_rows(oracle.scores(q, k, scale, False))[0]
    return dq, dk, np.swapaxes(p, -1, -2) @ np.asarray(do, dtype=np.float64)


MUTANTS = {
    "dS without the row term": _no_delta,
    "row term as a plain mean of dP": _delta_unweighted,
    "dK without the softmax scale": _dk_no_scale,
    "dQ from dS transposed": _dq_transposed,
    "dQ and dK with the wrong sign": _sign_flip,
    "dV from the unmasked P": _dv_unmasked,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutations(name):
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught += 1
    assert caught > 0, f"no pin catches: {name}"


def test_varlen_is_per_sequence():
    """A packed batch's gradients equal the dense gradients of each sequence,
    and keys of one sequence get nothing from another's queries."""
    rng = np.random.default_rng(12)
    H, d = 2, 4
    lq, lk = [3, 0, 5], [4, 2, 5]
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    q = rng.standard_normal((H, cu_q[-1], d))
    k = rng.standard_normal((H, cu_k[-1], d))
    v = rng.standard_normal((H, cu_k[-1], d))
    do = rng.standard_normal((H, cu_q[-1], d))
    for causal in (False, True):
        dq, dk, dv = BW.attention_backward_varlen(q, k, v, do, cu_q, cu_k, 0.6, causal)
        for s in range(3):
            sl_q, sl_k = slice(cu_q[s], cu_q[s + 1]), slice(cu_k[s], cu_k[s + 1])
            rq, rk, rv = BW.attention_backward(q[:, sl_q], k[:, sl_k], v[:, sl_k], do[:, sl_q], 0.6, causal)
            np.testing.assert_array_equal(dq[:, sl_q], rq)
            np.testing.assert_array_equal(dk[:, sl_k], rk)
            np.testing.assert_array_equal(dv[:, sl_k], rv)
        assert np.all(dk[:, cu_k[1]:cu_k[2]] == 0.0)  # sequence 1 has no queries
