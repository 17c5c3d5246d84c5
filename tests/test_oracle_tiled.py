"""Pins of the tiled online-softmax oracle (CPU only).

The blog's §2.2 claims the tiled recurrence gives the same result as the
one-shot softmax; these tests hold both recurrence forms to the one-shot
definition over many tile shapes, with and without the causal mask, and
with tiles that are entirely masked for some rows.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import tiled as T

RNG = np.random.default_rng(99)


@pytest.mark.parametrize("form", ["normalized", "deferred"])
@pytest.mark.parametrize("n", [1, 7, 128, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_one_shot(form, n, causal):
    d = 16
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    ref_o, ref_l = oracle.attention(q, k, v, 0.25, causal)
    for br, bc in itertools.product([1, 3, 16, 64, 128], [1, 3, 16, 64, 128]):
        if n > 128 and (br < 16 or bc < 16):
            continue  # keep the CPU suite short; small tiles are covered at n <= 128
        o, lse = oracle.attention_tiled(q, k, v, 0.25, causal, br, bc, form)
        np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


@pytest.mark.parametrize("form", ["normalized", "deferred"])
def test_masked_tiles_no_nan(form):
    """Nq != Nk and Br != Bc: some (row, tile) pairs are entirely masked."""
    q = RNG.standard_normal((37, 8)) * 4
    k = RNG.standard_normal((23, 8)) * 4
    v = RNG.standard_normal((23, 5))
    ref_o, ref_l = oracle.attention(q, k, v, 0.5, True)
    o, lse = oracle.attention_tiled(q, k, v, 0.5, True, br=5, bc=4, form=form)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(o, ref_o, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, atol=1e-12)


def test_tiled_large_logits():
    """Scores of magnitude ~1e3 (like outlier features): no overflow, same result."""
    q = RNG.standard_normal((40, 8)) * 40
    k = RNG.standard_normal((50, 8)) * 40
    v = RNG.standard_normal((50, 4))
    ref_o, ref_l = oracle.attention(q, k, v, 0.35, False)
    for form in ("normalized", "deferred"):
        o, lse = oracle.attention_tiled(q, k, v, 0.35, False, 16, 8, form)
        np.testing.assert_allclose(o, ref_o, atol=1e-12)
        np.testing.assert_allclose(lse, ref_l, rtol=1e-14, atol=1e-10)


def test_empty_keys():
    q = RNG.standard_normal((5, 4))
    o, lse = oracle.attention_tiled(q, q[:0], q[:0], 1.0, False, 2, 2)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_exp_diff_conventions():
    out = T._exp_diff(np.array([-np.inf, 0.0, -np.inf, 1.0]), np.array([-np.inf, -np.inf, 0.0, 2.0]))
    assert out[0] == 0 and out[1] == 0 and out[2] == 0
    assert out[3] == pytest.approx(np.exp(-1.0), abs=1e-16)


def test_mutation_missing_rescale(monkeypatch):
    """Planting a dropped e^{m_old - m_new} factor must break the equivalence."""
    def bad(a, b):
        return np.ones(np.broadcast(a, b).shape)
    monkeypatch.setattr(T, "_exp_diff", bad)
    q, k, v = (RNG.standard_normal((30, 8)) for _ in range(3))
    ref_o, _ = oracle.attention(q, k, v, 0.5, False)
    o, _ = oracle.attention_tiled(q, k, v, 0.5, False, 8, 8, "deferred")
    assert np.max(np.abs(o - ref_o)) > 1e-6
