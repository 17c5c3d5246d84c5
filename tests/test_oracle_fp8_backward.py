"""Pins of the fp8 backward oracle (CPU only).

``oracle.fp8_backward`` is held to things other than its own formulas:

* e5m2 rounding against torch's float8_e5m2 cast (an independent
  implementation of the OCP format) over every finite code, every midpoint
  between neighbouring codes and random values, and the bit patterns against
  torch's;
* the block quantisation of dO: the element of largest magnitude of each tile
  codes to +-57344, and dequantised values lie within half a code step;
* with rounding off, the fp8 backward must equal the exact gradients of the
  dequantised operands (``oracle.backward``, pinned on finite differences),
  whatever the tile scales: this catches a dropped term, a wrong sign or a
  transposed operand, and any fold factor that does not cancel;
* one visible key per row: P = 1, so dS = 0 (dQ = dK = 0 exactly) and
  dV = sum of the rows of dO, exactly when the dO scales are powers of two
  (the folded P codes are then exact), rounding on;
* with rounding on, the error against the exact gradients stays within
  what rounding P to 3 and dS to 2 mantissa bits can do.

``test_mutation_*`` plant mistakes into the oracle and check that a pin fails.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as BW
from oracle import fp8 as F8
from oracle import fp8_backward as FB


# --------------------------------------------------------------------- e5m2

def _all_finite_e5m2():
    codes = np.arange(256, dtype=np.uint8)
    vals = FB.e5m2_decode(codes)
    return codes[np.isfinite(vals)], vals[np.isfinite(vals)]


def _torch_e5m2(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e5m2).to(torch.float64).numpy()


def test_e5m2_codes_match_torch():
    codes, vals = _all_finite_e5m2()
    assert len(codes) == 248  # 256 minus +-inf and 6 NaNs
    t = torch.tensor(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals, t)
    assert vals.max() == 57344.0 and np.min(vals[vals > 0]) == 2.0 ** -16
    # encode is the inverse of decode on every finite code
    np.testing.assert_array_equal(FB.e5m2_encode(vals) & 0x7F, codes & 0x7F)


def test_e5m2_round_matches_torch_on_codes_midpoints_and_random():
    _, vals = _all_finite_e5m2()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2  # ties: to the even code
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.standard_normal(20000) * s for s in (1e-5, 1e-3, 1.0, 1e2, 1e4)])
    x = np.concatenate([vals, mids, -mids, rnd[np.abs(rnd) < 57344]]).astype(np.float32)
    np.testing.assert_array_equal(FB.e5m2_round_f32(x), _torch_e5m2(x))


def test_e5m2_saturates():
    np.testing.assert_array_equal(FB.e5m2_round(np.array([6e4, -1e9, 57344.0])), [57344.0, -57344.0, 57344.0])


def test_quantize_e5m2_tiles():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 300, 16)) * np.exp(rng.standard_normal((2, 3, 300, 1)))
    x[0, 1, 128:256] = 0.0  # an all-zero tile takes scale 1
    codes, s = FB.quantize_e5m2(x)
    assert s.shape == (2, 3, 3) and s.dtype == np.float32
    assert s[0, 1, 1] == 1.0
    back = FB.dequantize_e5m2(codes, s)
    for t in range(3):
        blk = x[..., t * 128:(t + 1) * 128, :]
        got = FB.e5m2_decode(codes[..., t * 128:(t + 1) * 128, :])
        amax_codes = np.abs(got).reshape(2, 3, -1).max(axis=-1)
        nz = np.abs(blk).reshape(2, 3, -1).max(axis=-1) > 0
        np.testing.assert_array_equal(amax_codes[nz], 57344.0)
        # half a code step: 2^-3 relative for normal codes, 2^-17 scaled below
        err = np.abs(back[..., t * 128:(t + 1) * 128, :] - blk)
        bound = np.maximum(np.abs(blk) * 2.0 ** -3, s[..., t, None, None] * 2.0 ** -17) * (1 + 1e-6)
        assert np.all(err <= bound)


# ------------------------------------------------------------- fp8 backward

def _fp8_problem(lead, nq, nk, d, seed, pow2_do=False, causal=False, scale=0.3):
    """e4m3 codes/scales for Q, K, V (rotation off), the exact forward of the
    dequantised operands (O, lse) and a dO."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(lead + (nq, d)) * np.exp(0.5 * rng.standard_normal(lead + (nq, 1)))
    k = rng.standard_normal(lead + (nk, d))
    v = rng.standard_normal(lead + (nk, d)) * np.exp(0.5 * rng.standard_normal(lead + (nk, 1)))
    q8, sq = F8.quantize(q)
    k8, sk = F8.quantize(k)
    v8, sv = F8.quantize(v)
    qd, kd, vd = F8.dequantize(q8, sq), F8.dequantize(k8, sk), F8.dequantize(v8, sv)
    o, lse = oracle.attention(qd, kd, vd, scale, causal)
    do = rng.standard_normal(lead + (nq, d))
    if pow2_do:
        # dO exactly representable, each tile's largest element at 57344 * 2^e:
        # its scales are then powers of two and quantisation is exact
        ntile = (nq + 127) // 128
        e = rng.integers(-9, -2, size=lead + (ntile,))
        do = FB.e5m2_round(do * 8000.0)
        for t in range(ntile):
            blk = do[..., t * 128:(t + 1) * 128, :]
            blk.reshape(lead + (-1,))[..., 0] = 57344.0
            do[..., t * 128:(t + 1) * 128, :] = blk * np.ldexp(1.0, e[..., t])[..., None, None]
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv, o=o, lse=lse, dout=do, qd=qd, kd=kd, vd=vd)


def pin_exact_without_rounding(bwd):
    for causal in (False, True):
        for nq, nk in ((300, 260), (129, 400), (64, 64)):
            pr = _fp8_problem((2,), nq, nk, 16, seed=nq + nk + causal, pow2_do=True, causal=causal)
            got = bwd(pr["q8"], pr["sq"], pr["k8"], pr["sk"], pr["v8"], pr["sv"], pr["o"], pr["lse"], pr["dout"],
                      0.3, causal, rounding=False)
            ref = BW.attention_backward(pr["qd"], pr["kd"], pr["vd"], pr["dout"], 0.3, causal)
            for g, r in zip(got, ref):
                np.testing.assert_allclose(g, r, rtol=1e-9, atol=1e-11 * np.abs(r).max())


def pin_single_key(bwd):
    # Nk = 1: every row's P is 1, dS = P (dP - dO.O) = 0 since O = v_0
    pr = _fp8_problem((3,), 400, 1, 16, seed=7, pow2_do=True)
    dq, dk, dv = bwd(pr["q8"], pr["sq"], pr["k8"], pr["sk"], pr["v8"], pr["sv"], pr["o"], pr["lse"], pr["dout"],
                     0.3, False, rounding=True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_array_equal(dv[..., 0, :], pr["dout"].sum(axis=-2))


def pin_rounding_error(bwd):
    pr = _fp8_problem((2,), 256, 384, 64, seed=3, scale=0.125)
    a = bwd(pr["q8"], pr["sq"], pr["k8"], pr["sk"], pr["v8"], pr["sv"], pr["o"], pr["lse"], pr["dout"], 0.125, False,
            rounding=True)
    b = bwd(pr["q8"], pr["sq"], pr["k8"], pr["sk"], pr["v8"], pr["sv"], pr["o"], pr["lse"], pr["dout"], 0.125, False,
            rounding=False)
    # relative RMSE below half a code step: P to 3 mantissa bits (dV), dS to 2 (dQ, dK)
    for g, r, bound in zip(a, b, (2.0 ** -3, 2.0 ** -3, 2.0 ** -4)):
        rel = np.sqrt(np.mean((g - r) ** 2)) / np.sqrt(np.mean(r ** 2))
        assert 0 < rel < bound


def test_fp8_backward_exact_without_rounding():
    pin_exact_without_rounding(FB.backward_fp8)


def test_fp8_backward_single_key():
    pin_single_key(FB.backward_fp8)


def test_fp8_backward_rounding_error():
    pin_rounding_error(FB.backward_fp8)


def test_fp8_backward_parts_and_codes_in_range():
    pr = _fp8_problem((2,), 200, 300, 32, seed=11, causal=True, scale=0.2)
    parts = FB.backward_fp8(pr["q8"], pr["sq"], pr["k8"], pr["sk"], pr["v8"], pr["sv"], pr["o"], pr["lse"],
                            pr["dout"], 0.2, True, parts=True)
    assert np.max(parts["p8"]) <= 256.0 and np.min(parts["p8"]) >= 0.0
    assert np.max(np.abs(parts["dsq"])) < FB.E5M2_MAX and np.max(np.abs(parts["dsk"])) < FB.E5M2_MAX
    # masked entries (key above the diagonal) contribute nothing
    nq, nk = 200, 300
    mask = np.arange(nk)[None, :] > np.arange(nq)[:, None]
    assert np.all(parts["P"][..., mask] == 0) and np.all(parts["dsq"][..., mask] == 0)


# ---------------------------------------------------------------- mutations

def test_mutation_p_scale(monkeypatch):
    monkeypatch.setattr(FB, "P_SCALE", 512.0)  # 2^9 P leaves e4m3's range: 512 saturates at 448
    with pytest.raises(AssertionError):
        pin_single_key(FB.backward_fp8)


def test_mutation_delta_sign(monkeypatch):
    orig = FB.backward_fp8

    def mutant(*a, **kw):
        pr = a[6]
        return orig(*a[:6], -np.asarray(pr), *a[7:], **kw)  # uses -O: delta of the wrong sign

    with pytest.raises(AssertionError):
        pin_exact_without_rounding(mutant)


def test_mutation_fold_not_cancelled(monkeypatch):
    # a fold ratio applied to the rounded factor but not undone in the product
    orig_rs = FB._row_scales
    monkeypatch.setattr(FB, "_row_scales", lambda s, n, t: orig_rs(s, n, t) * 2.0)
    with pytest.raises(AssertionError):
        pin_exact_without_rounding(FB.backward_fp8)


def test_mutation_e5m2_mantissa(monkeypatch):
    monkeypatch.setattr(FB, "E5M2_MANT_BITS", 3)
    with pytest.raises(AssertionError):
        test_e5m2_round_matches_torch_on_codes_midpoints_and_random()
