"""Pins of the attention oracle (CPU only).

Each check compares the oracle with something other than itself: a brute
force triple loop, closed forms, invariants, and torch's CPU attention in
float64 for the special case it covers.  ``test_mutations`` plants plausible
mistakes into the oracle (on the CPU) and asserts that some pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import exact as A
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def brute_force(q, k, v, scale, causal):
    """Pure-Python loops: the definition written out element by element."""
    nq, d = len(q), len(q[0])
    nk = len(k)
    o = [[0.0] * len(v[0]) if nk else [0.0] * d for _ in range(nq)]
    lse = [-math.inf] * nq
    for i in range(nq):
        s = []
        for j in range(nk):
            if causal and j > i:
                continue
            s.append((j, scale * sum(q[i][t] * k[j][t] for t in range(d))))
        if not s:
            continue
        m = max(x for _, x in s)
        e = [(j, math.exp(x - m)) for j, x in s]
        l = sum(x for _, x in e)
        lse[i] = m + math.log(l)
        for c in range(len(v[0])):
            o[i][c] = sum(w * v[j][c] for j, w in e) / l
    return np.array(o), np.array(lse)


# ---------------------------------------------------------------- pin checks
# Each returns normally or raises AssertionError; the mutation test reuses them.

def check_brute_force():
    for (nq, nk, d, causal) in [(5, 7, 3, False), (7, 5, 4, True), (8, 8, 8, True), (3, 1, 2, False), (6, 6, 5, True)]:
        q, k, v = (RNG.standard_normal((n, d)) for n in (nq, nk, nk))
        o, lse = oracle.attention(q, k, v, 0.37, causal)
        ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.37, causal)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def check_torch_sdpa():
    for (B, H, nq, nk, d, causal) in [(2, 3, 33, 33, 16, False), (1, 2, 40, 40, 8, True), (1, 1, 17, 29, 8, True), (2, 1, 29, 17, 4, True)]:
        q, k, v = (RNG.standard_normal((B, H, n, d)) for n in (nq, nk, nk))
        scale = 1.0 / math.sqrt(d) * 1.3
        o, lse = oracle.attention(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        s = scale * tq @ tk.transpose(-1, -2)
        if causal:
            s = s.masked_fill(~torch.ones(nq, nk, dtype=torch.bool).tril(), -math.inf)
        lt = torch.logsumexp(s, dim=-1)
        np.testing.assert_allclose(o, ot.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lt.numpy(), rtol=0, atol=1e-12)


def check_rows_sum_to_one():
    s = oracle.scores(RNG.standard_normal((2, 19, 8)), RNG.standard_normal((2, 23, 8)), 0.5, causal=True)
    p, _, _ = oracle.softmax_rows(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    hidden = np.arange(23)[None, :] > np.arange(19)[:, None]
    assert np.all(p[:, hidden] == 0)


def check_shift_invariance():
    q, k, v = RNG.standard_normal((11, 6)), RNG.standard_normal((13, 6)), RNG.standard_normal((13, 5))
    scale = 0.4
    # (a) at the score level: S_i += c_i
    s = oracle.scores(q, k, scale)
    c = RNG.standard_normal(11)[:, None] * 30.0
    p1, m1, l1 = oracle.softmax_rows(s)
    p2, m2, l2 = oracle.softmax_rows(s + c)
    np.testing.assert_allclose(p1 @ v, p2 @ v, atol=1e-12)
    np.testing.assert_allclose((m2 + np.log(l2)) - (m1 + np.log(l1)), c[:, 0], atol=1e-12)
    # (b) through the inputs: K_j += w adds scale * q_i . w to every score of row i
    w = RNG.standard_normal(6) * 3
    o1, lse1 = oracle.attention(q, k, v, scale)
    o2, lse2 = oracle.attention(q, k + w, v, scale)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse1, scale * q @ w, atol=1e-12)


def check_identical_keys():
    nq, nk, d = 9, 12, 4
    q = RNG.standard_normal((nq, d))
    k = np.repeat(RNG.standard_normal((1, d)), nk, axis=0)
    v = RNG.standard_normal((nk, 3))
    scale = 0.7
    s_i = scale * q @ k[0]
    o, lse = oracle.attention(q, k, v, scale)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), atol=1e-12)
    np.testing.assert_allclose(lse, s_i + math.log(nk), atol=1e-12)
    oc, lsec = oracle.attention(q, k, v, scale, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, nk + 1)[:, None]
    np.testing.assert_allclose(oc, prefix[:nq], atol=1e-12)
    np.testing.assert_allclose(lsec, s_i + np.log(np.arange(1, nq + 1)), atol=1e-12)


def check_masked_prefix():
    q, k, v = RNG.standard_normal((6, 4)), RNG.standard_normal((6, 4)), RNG.standard_normal((6, 4))
    o, lse = oracle.attention(q, k, v, 0.9, causal=True)
    # row 0 sees only key 0: O_0 = V_0 exactly, lse_0 = S_00
    assert np.array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(0.9 * q[0] @ k[0], abs=1e-15)
    # no key at all: O = 0, lse = -inf, no NaN
    o0, l0 = oracle.attention(q, k[:0], v[:0], 0.9, causal=True)
    assert np.all(o0 == 0) and np.all(l0 == -np.inf)
    o0, l0 = oracle.attention(q, k[:0], v[:0], 0.9, causal=False)
    assert np.all(o0 == 0) and np.all(l0 == -np.inf)


def check_closed_forms():
    q, k, v = RNG.standard_normal((5, 3)), RNG.standard_normal((2, 3)), RNG.standard_normal((2, 4))
    scale = 1.1
    # one key: O = V_0, lse = s
    o, lse = oracle.attention(q, k[:1], v[:1], scale)
    np.testing.assert_allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-15)
    np.testing.assert_allclose(lse, scale * q @ k[0], atol=1e-14)
    # two keys: weight of key 0 is sigmoid(s0 - s1)
    o, lse = oracle.attention(q, k, v, scale)
    s0, s1 = scale * q @ k[0], scale * q @ k[1]
    w0 = 1.0 / (1.0 + np.exp(-(s0 - s1)))
    np.testing.assert_allclose(o, w0[:, None] * v[0] + (1 - w0)[:, None] * v[1], atol=1e-13)
    np.testing.assert_allclose(lse, np.logaddexp(s0, s1), atol=1e-13)
    # Q = 0: uniform weights, lse = ln Nk
    vv = RNG.standard_normal((7, 4))
    o, lse = oracle.attention(np.zeros((3, 3)), RNG.standard_normal((7, 3)), vv, scale)
    np.testing.assert_allclose(o, np.broadcast_to(vv.mean(0), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(7), atol=1e-14)


def check_varlen_is_concatenation():
    lengths = [3, 0, 5, 1, 4]
    cu = W.cu_seqlens(lengths)
    T, H, d = int(cu[-1]), 2, 4
    q, k, v = (RNG.standard_normal((H, T, d)) for _ in range(3))
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cu, cu, 0.5, causal)
        for b in range(len(lengths)):
            sl = slice(cu[b], cu[b + 1])
            ob, lb = oracle.attention(q[:, sl], k[:, sl], v[:, sl], 0.5, causal)
            assert np.array_equal(o[:, sl], ob) and np.array_equal(lse[:, sl], lb)
    # different q and k lengths per sequence (top-left causal per sequence)
    cq, ck = W.cu_seqlens([2, 4]), W.cu_seqlens([3, 1])
    q2 = RNG.standard_normal((H, 6, d))
    k2, v2 = RNG.standard_normal((H, 4, d)), RNG.standard_normal((H, 4, d))
    o, lse = oracle.attention_varlen(q2, k2, v2, cq, ck, 0.5, True)
    ob, lb = brute_force(q2[0, 2:6].tolist(), k2[0, 3:4].tolist(), v2[0, 3:4].tolist(), 0.5, True)
    np.testing.assert_allclose(o[0, 2:6], ob, atol=1e-13)
    np.testing.assert_allclose(lse[0, 2:6], lb, atol=1e-13)


def check_rows_helper():
    q, k, v = RNG.standard_normal((20, 8)), RNG.standard_normal((25, 8)), RNG.standard_normal((25, 8))
    rows = [0, 3, 19, 7]
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.3, causal)
        orow, lrow = A.attention_rows(q, k, v, rows, 0.3, causal)
        np.testing.assert_allclose(orow, o[rows], atol=1e-13)
        np.testing.assert_allclose(lrow, lse[rows], atol=1e-13)


def check_repeated_pairs():
    """Every (key, value) pair repeated m times, in any order: the softmax
    weights of the copies of one pair add up to that pair's weight, so O is
    unchanged and every row sum is m times larger (lse + ln m).  The
    full-size GPU test of key offsets beyond 2^31 elements relies on it."""
    q, k, v = RNG.standard_normal((7, 5)), RNG.standard_normal((11, 5)), RNG.standard_normal((11, 3))
    m = 4
    perm = RNG.permutation(11 * m)
    kr, vr = np.tile(k, (m, 1))[perm], np.tile(v, (m, 1))[perm]
    o, lse = oracle.attention(q, k, v, 0.6)
    o_r, lse_r = oracle.attention(q, kr, vr, 0.6)
    np.testing.assert_allclose(o_r, o, atol=1e-13)
    np.testing.assert_allclose(lse_r, lse + math.log(m), atol=1e-13)


PINS = [check_brute_force, check_torch_sdpa, check_rows_sum_to_one, check_shift_invariance,
        check_identical_keys, check_masked_prefix, check_closed_forms, check_varlen_is_concatenation,
        check_rows_helper, check_repeated_pairs]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_golden_cu_seqlens():
    g = json.load(open(os.path.join(GOLDEN, "cu_seqlens_example.json")))
    assert W.cu_seqlens(g["lengths"]).tolist() == g["cu_seqlens"]


def test_golden_flop_ratio():
    g = json.load(open(os.path.join(GOLDEN, "flop_ratio.json")))
    # FLOPs per score element (two contractions of 2*d) over one exponential per element
    w = W.Workload("x", 1, 1, 10, 10, g["head_dim"], "bf16", False)
    assert w.flops() / (w.Nq * w.Nk) == g["matmul_flops_per_exp"]
    assert round(100 * g["fa3_fp16_tflops"] / g["h100_fp16_peak_tflops"]) == g["utilization_percent"]
    wc = W.Workload("x", 1, 1, 10, 10, 128, "bf16", True)
    assert wc.flops() == w.flops() / 2


# ---------------------------------------------------------------- mutations

def _mut_scores_no_scale(q, k, scale, causal=False):
    return ORIG_SCORES(q, k, 1.0, causal)


def _mut_scores_wrong_mask(q, k, scale, causal=False):
    s = ORIG_SCORES(q, k, scale, False)
    if causal:
        i = np.arange(s.shape[-2])[:, None]
        j = np.arange(s.shape[-1])[None, :]
        s = np.where(j < i, s, -np.inf)  # off by one: drops the diagonal
    return s


def _mut_scores_bottom_right(q, k, scale, causal=False):
    s = ORIG_SCORES(q, k, scale, False)
    if causal:
        nq, nk = s.shape[-2], s.shape[-1]
        i = np.arange(nq)[:, None]
        j = np.arange(nk)[None, :]
        s = np.where(j <= i + (nk - nq), s, -np.inf)
    return s


def _mut_softmax_no_max(s):
    p, m, l = ORIG_SOFTMAX(s)
    return p, np.zeros_like(m), l  # forgets the max in lse


def _mut_softmax_transposed(s):
    p, m, l = ORIG_SOFTMAX(s)
    if p.shape[-1] == p.shape[-2]:
        p = np.swapaxes(p, -1, -2)
    return p, m, l


ORIG_SCORES = A.scores
ORIG_SOFTMAX = A.softmax_rows


@pytest.mark.parametrize("target,mutant", [
    ("scores", _mut_scores_no_scale),
    ("scores", _mut_scores_wrong_mask),
    ("scores", _mut_scores_bottom_right),
    ("softmax_rows", _mut_softmax_no_max),
    ("softmax_rows", _mut_softmax_transposed),
])
def test_mutations(monkeypatch, target, mutant):
    """A planted mistake in the oracle must make at least one pin fail."""
    monkeypatch.setattr(A, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutation {mutant.__name__} was not caught by any pin"
