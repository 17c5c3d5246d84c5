"""Pins of the split-KV oracle and the (O, lse) merge (CPU only).

The split computation is held to the full attention of ``oracle.exact`` (a
different code path: one softmax over all keys), to element-by-element loops
over each key chunk, to a two-key closed form, and to invariants of the
merge (order, a single part, empty parts, large scores).  ``test_mutations``
plants plausible mistakes into copies of the functions and checks that some
pin catches each.
"""

import math
import types

import numpy as np
import pytest

import oracle
from oracle import splitkv as SK

RNG = np.random.default_rng(4321)


def _problem(shape_q, nk, d, scale_mag=1.0, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape_q + (d,)) * scale_mag
    k = rng.standard_normal(shape_q[:-1] + (nk, d))
    v = rng.standard_normal(shape_q[:-1] + (nk, d))
    return q, k, v


def chunk_loops(q, k, v, scale, causal, kb, ke):
    """The partial result of one chunk, written out with Python loops."""
    nq, d = q.shape
    o = np.zeros((nq, v.shape[1]))
    lse = np.full(nq, -math.inf)
    for i in range(nq):
        s = [(j, scale * sum(q[i, t] * k[j, t] for t in range(d))) for j in range(kb, ke) if not (causal and j > i)]
        if not s:
            continue
        m = max(x for _, x in s)
        e = [(j, math.exp(x - m)) for j, x in s]
        l = sum(x for _, x in e)
        lse[i] = m + math.log(l)
        for c in range(v.shape[1]):
            o[i, c] = sum(w * v[j, c] for j, w in e) / l
    return o, lse


# ---------------------------------------------------------------- pin checks
# Each takes the module under test (the oracle, or a mutated copy).

def pin_equals_full(mod):
    for causal in (False, True):
        for nq, nk in ((7, 13), (16, 16), (5, 40)):
            q, k, v = _problem((2, 3, nq), nk, 8, seed=nq * 100 + nk)
            ref_o, ref_l = oracle.attention(q, k, v, 0.35, causal)
            for ns in (1, 2, 3, 5, 8, nk + 3):
                o, lse = mod.attention_splitkv(q, k, v, 0.35, causal, ns)
                np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def pin_chunks_by_loops(mod):
    q, k, v = _problem((6,), 11, 4, seed=7)
    for causal in (False, True):
        for kb, ke in ((0, 4), (4, 8), (8, 11), (3, 3), (5, 11)):
            o, lse = mod.attention_partial(q, k, v, 0.5, causal, kb, ke)
            ro, rl = chunk_loops(q, k, v, 0.5, causal, kb, ke)
            np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
            assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
            fin = np.isfinite(rl)
            np.testing.assert_allclose(lse[fin], rl[fin], rtol=0, atol=1e-12)


def pin_two_key_closed_form(mod):
    # one query, two keys; scores a and b land in different chunks
    a, b = 0.7, -1.9
    q = np.array([[1.0, 0.0]])
    k = np.array([[a, 5.0], [b, -3.0]])
    v = np.array([[2.0, -1.0, 0.5], [-4.0, 3.0, 1.5]])
    o, lse = mod.attention_splitkv(q, k, v, 1.0, False, 2)
    ea, eb = math.exp(a), math.exp(b)
    np.testing.assert_allclose(o[0], (ea * v[0] + eb * v[1]) / (ea + eb), rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse[0], math.log(ea + eb), rtol=1e-14, atol=0)


def pin_merge_invariants(mod):
    rng = np.random.default_rng(11)
    o_parts = rng.standard_normal((4, 3, 5, 6))
    lse_parts = rng.standard_normal((4, 3, 5)) * 3
    lse_parts[2, 1, :] = -np.inf  # an empty chunk for some rows
    o_parts[2, 1, :] = 0.0
    o, lse = mod.merge(o_parts, lse_parts)
    perm = [3, 0, 2, 1]
    o2, lse2 = mod.merge(o_parts[perm], lse_parts[perm])
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    o1, l1 = mod.merge(o_parts[:1], lse_parts[:1])
    np.testing.assert_allclose(o1, o_parts[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l1, lse_parts[0], rtol=0, atol=1e-15)
    # lse is the log-sum-exp of the parts, written out per row
    for i in range(3):
        for j in range(5):
            vals = [x for x in lse_parts[:, i, j] if np.isfinite(x)]
            np.testing.assert_allclose(lse[i, j], math.log(sum(math.exp(x) for x in vals)), rtol=1e-13)


def pin_empty_and_masked(mod):
    q, k, v = _problem((4,), 3, 5, seed=3)
    # more chunks than keys: empty chunks carry no weight
    o, lse, op, lp = mod.attention_splitkv(q, k, v, 0.4, False, 6, parts=True)
    assert np.all(np.isneginf(lp[3:])) and np.all(op[3:] == 0.0)
    ref_o, ref_l = oracle.attention(q, k, v, 0.4, False)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-13)
    # causal: query 0 sees only key 0, so the chunk [1, 3) is empty for it
    o, lse, op, lp = mod.attention_splitkv(q, k, v, 0.4, True, 2, parts=True)
    assert np.isneginf(lp[1, 0]) and np.all(op[1, 0] == 0.0)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-14)
    # no keys at all
    o, lse = mod.attention_splitkv(q, k[:0], v[:0], 0.4, False, 3)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def pin_large_scores(mod):
    # lse beyond 709: e^{lse} overflows fp64, the merge must not
    q, k, v = _problem((3, 9), 20, 6, scale_mag=30.0, seed=5)
    ref_o, ref_l = oracle.attention(q, k, v, 4.0, False)
    assert np.max(ref_l) > 720  # e^720 is beyond fp64
    o, lse = mod.attention_splitkv(q, k, v, 4.0, False, 4)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-14, atol=0)


PINS = [pin_equals_full, pin_chunks_by_loops, pin_two_key_closed_form, pin_merge_invariants,
        pin_empty_and_masked, pin_large_scores]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(SK)


def test_split_bounds():
    assert SK.split_bounds(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert SK.split_bounds(2, 4) == [(0, 1), (1, 2), (2, 2), (2, 2)]
    assert SK.split_bounds(0, 2) == [(0, 0), (0, 0)]
    for nk in range(0, 40):
        for ns in range(1, 9):
            b = SK.split_bounds(nk, ns)
            assert len(b) == ns and b[0][0] == 0 and b[-1][1] == nk
            assert all(b[i][1] == b[i + 1][0] for i in range(ns - 1))


# ---------------------------------------------------------------- mutations

def _mutant(**over):
    m = types.SimpleNamespace(**{n: getattr(SK, n) for n in ("split_bounds", "attention_partial", "merge",
                                                              "attention_splitkv")})
    for k, f in over.items():
        setattr(m, k, f)

    def attention_splitkv(q, k, v, scale, causal, num_splits, parts=False):
        nk = np.asarray(k).shape[-2]
        outs = [m.attention_partial(q, k, v, scale, causal, b, e) for b, e in m.split_bounds(nk, num_splits)]
        op = np.stack([o for o, _ in outs])
        lp = np.stack([l for _, l in outs])
        o, lse = m.merge(op, lp)
        return (o, lse, op, lp) if parts else (o, lse)

    if "attention_splitkv" not in over:
        m.attention_splitkv = attention_splitkv
    return m


def _merge_no_shift(o_parts, lse_parts):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        w = np.exp(lse_parts)
        tot = w.sum(0)
        return (w[..., None] * o_parts).sum(0) / tot[..., None], np.log(tot)


def _merge_unnormalised(o_parts, lse_parts):
    m = lse_parts.max(0)
    w = np.exp(lse_parts - m[None])
    return (w[..., None] * o_parts).sum(0), m + np.log(w.sum(0))


def _merge_linear(o_parts, lse_parts):
    w = np.where(np.isfinite(lse_parts), lse_parts - lse_parts.min(0)[None] + 1.0, 0.0)
    return (w[..., None] * o_parts).sum(0) / w.sum(0)[..., None], lse_parts.max(0)


def _bounds_overlap(nk, ns):
    n = -(-nk // ns) if nk > 0 else 0
    return [(max(0, min(s * n - 1, nk)), min((s + 1) * n, nk)) for s in range(ns)]


def _partial_local_causal(q, k, v, scale, causal, kb, ke):
    return oracle.attention(np.asarray(q), np.asarray(k)[..., kb:ke, :], np.asarray(v)[..., kb:ke, :], scale, causal)


MUTANTS = {
    "merge without the max shift": dict(merge=_merge_no_shift),
    "merge without normalisation": dict(merge=_merge_unnormalised),
    "merge with linear weights": dict(merge=_merge_linear),
    "overlapping chunks": dict(split_bounds=_bounds_overlap),
    "causal mask with chunk-local indices": dict(attention_partial=_partial_local_causal),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutations(name):
    mod = _mutant(**MUTANTS[name])
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, FloatingPointError):
            caught += 1
    assert caught > 0, f"no pin catches: {name}"
