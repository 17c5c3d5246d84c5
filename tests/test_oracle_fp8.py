"""Pins of the fp8 oracle pieces (CPU only).

* e4m3 rounding and codes against torch's float8_e4m3fn (a library routine),
  bit for bit, plus the format's boundary values;
* the Sylvester Hadamard matrix (H H^T = d I in integers), the fast
  transform against the matrix, and (QM)(KM)^T = QK^T;
* quantisation by its defining properties (amax element -> 448, round to
  nearest code, per-tile independence);
* fp8 attention: with P unrounded it reduces to plain attention on the
  dequantised inputs; with P rounded it stays within the rounding bound;
* the method-level claim of the wiki page ("Three techniques" §3): with
  outlier channels, block scales plus incoherent processing give a lower
  RMSE than one scale per tensor.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
import workloads as W

RNG = np.random.default_rng(7)


# ------------------------------------------------------------------ e4m3

def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_encode_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(F.e4m3_encode(vals[fin]), codes[fin])


def test_round_matches_torch_cast_sweep():
    mag = np.exp2(RNG.uniform(-14, np.log2(464), 400000))
    x = (mag * RNG.choice([-1.0, 1.0], mag.shape)).astype(np.float32)
    # every e4m3 value and every midpoint between neighbours, both signs
    grid = np.unique(np.abs(F.e4m3_decode(np.arange(127, dtype=np.uint8))))
    mids = (grid[:-1] + grid[1:]) / 2
    x = np.concatenate([x, grid, -grid, mids, -mids]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    ours = F.e4m3_round_f32(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(ours, ref.astype(np.float64))


@pytest.mark.parametrize("x,expected", [
    (448.0, 448.0), (464.0, 448.0),  # 464 is the tie between 448 and 480: even mantissa wins
    (470.0, 448.0), (1e9, 448.0),  # saturation (the oracle's reading; torch gives NaN here)
    (2.0 ** -9, 2.0 ** -9), (2.0 ** -10, 0.0), (3 * 2.0 ** -11, 2.0 ** -9),
    (17.0, 16.0), (18.0, 18.0), (19.0, 20.0), (-0.0, -0.0), (2.0 ** -6, 2.0 ** -6),
])
def test_round_boundaries(x, expected):
    r = float(F.e4m3_round(np.float64(x)))
    assert r == expected and np.signbit(r) == np.signbit(expected)


# ------------------------------------------------------------------ Hadamard

@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_sylvester_orthogonal_integers(d):
    h = F.sylvester(d)
    assert h.dtype == np.int64 and set(np.unique(h)) <= {-1, 1}
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)


@pytest.mark.parametrize("d", [2, 64, 128, 256])
def test_fwht_equals_matrix(d):
    x = RNG.standard_normal((5, d))
    np.testing.assert_allclose(F.fwht(x), x @ F.sylvester(d), rtol=0, atol=1e-12 * np.sqrt(d) * 8)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_preserves_scores(d):
    s = RNG.choice([-1.0, 1.0], d)
    m = F.rotation_matrix(s)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-14)
    q = RNG.standard_normal((33, d)) * np.where(np.arange(d) < 4, 50, 1)
    k = RNG.standard_normal((40, d)) * np.where(np.arange(d) < 4, 50, 1)
    qk = q @ k.T
    rot = F.rotate(q, s) @ F.rotate(k, s).T
    assert np.max(np.abs(rot - qk)) <= 1e-12 * np.max(np.abs(qk))


# ------------------------------------------------------------------ quantisation

def _check_quantized(x_rot, codes, scales, tile, per_tensor):
    vals = F.e4m3_decode(codes)
    n = x_rot.shape[-2]
    rs = np.repeat(scales.astype(np.float64), tile, axis=-1)[..., :n][..., None]
    y = (x_rot.astype(np.float32) / rs.astype(np.float32)).astype(np.float64)
    # round to nearest: no other code is closer to y than the chosen one
    grid = np.unique(F.e4m3_decode(np.arange(256, dtype=np.uint8)))
    grid = grid[~np.isnan(grid)]
    idx = np.clip(np.searchsorted(grid, y), 1, len(grid) - 1)
    best = np.minimum(np.abs(grid[idx] - y), np.abs(grid[idx - 1] - y))
    assert np.all(np.abs(vals - y) <= best)
    # the largest magnitude of each tile (or of the tensor) lands on 448
    if per_tensor:
        assert np.max(np.abs(vals)) == 448.0
        assert np.all(scales == scales.flat[0])
    else:
        for t in range(scales.shape[-1]):
            blk = np.abs(vals[..., t * tile:(t + 1) * tile, :]).reshape(vals.shape[:-2] + (-1,))
            xb = np.abs(x_rot[..., t * tile:(t + 1) * tile, :]).reshape(vals.shape[:-2] + (-1,))
            nz = xb.max(axis=-1) > 0
            assert np.all(blk.max(axis=-1)[nz] == 448.0)
            assert np.all(scales[..., t][~nz] == 1.0)


@pytest.mark.parametrize("per_tensor", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_properties(per_tensor, rotate):
    d, n = 64, 300  # three 128-row tiles, the last one ragged
    x = RNG.standard_normal((2, 3, n, d)).astype(np.float32) * np.exp(RNG.uniform(-3, 3, (2, 3, 1, 1))).astype(np.float32)
    x[1, 2, 128:256] = 0.0  # an all-zero tile
    s = RNG.choice([-1.0, 1.0], d).astype(np.float32) if rotate else None
    codes, scales = F.quantize(x, s, per_tensor)
    assert codes.dtype == np.uint8 and codes.shape == x.shape
    assert scales.dtype == np.float32 and scales.shape == (2, 3, 3)
    x_rot = F.rotate(x, s) if rotate else x.astype(np.float64)
    _check_quantized(x_rot, codes, scales, 128, per_tensor)
    # dequantisation error: half a spacing of the binade, relative 2^-4 (normals)
    deq = F.dequantize(codes, scales)
    rs = np.repeat(scales.astype(np.float64), 128, axis=-1)[..., :n][..., None]
    assert np.all(np.abs(deq - x_rot) <= np.maximum(2.0 ** -4 * np.abs(x_rot), rs * 2.0 ** -10) * (1 + 1e-6))


def test_quantize_tiles_independent():
    x = RNG.standard_normal((1, 1, 256, 64)).astype(np.float32)
    _, s1 = F.quantize(x)
    x2 = x.copy()
    x2[0, 0, 200, 5] = 1000.0
    _, s2 = F.quantize(x2)
    assert s1[0, 0, 0] == s2[0, 0, 0] and s2[0, 0, 1] > s1[0, 0, 1]


# ------------------------------------------------------------------ fp8 attention

def _codes_problem(nq, nk, d, seed):
    q8 = W.random_e4m3_codes((2, nq, d), seed, max_exp_field=9)
    k8 = W.random_e4m3_codes((2, nk, d), seed + 1, max_exp_field=9)
    v8 = W.random_e4m3_codes((2, nk, d), seed + 2, max_exp_field=9)
    nt = lambda n: (n + 127) // 128  # noqa: E731
    sq = W.random_scales((2, nt(nq)), seed + 3)
    sk = W.random_scales((2, nt(nk)), seed + 4)
    sv = W.random_scales((2, nt(nk)), seed + 5)
    return q8, k8, v8, sq, sk, sv


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_reduces_to_plain(causal):
    q8, k8, v8, sq, sk, sv = _codes_problem(200, 300, 32, 11)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal, quantize_p=False)
    ref_o, ref_l = oracle.attention(F.dequantize(q8, sq), F.dequantize(k8, sk), F.dequantize(v8, sv), 0.3, causal)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_p_rounding_bound(causal):
    q8, k8, v8, sq, sk, sv = _codes_problem(150, 260, 32, 21)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal)
    o_exact, lse_exact = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal, quantize_p=False)
    assert not np.allclose(o, o_exact, atol=1e-9)  # P really is rounded
    np.testing.assert_allclose(lse, lse_exact, rtol=0, atol=1e-12)  # l uses unrounded p
    # bound: each weight moves by <= 2^-4 relative, or <= 2^-10 * 2^-8 absolute (subnormal codes)
    qd, kd, vd = F.dequantize(q8, sq), F.dequantize(k8, sk), F.dequantize(v8, sv)
    p, _, _ = oracle.softmax_rows(oracle.scores(qd, kd, 0.3, causal))
    bound = (2.0 ** -4 * p + 2.0 ** -18) @ np.abs(vd) * 1.000001
    assert np.all(np.abs(o - o_exact) <= bound + 1e-12)


def test_fp8_power_of_two_invariance():
    """Doubling every V scale doubles O exactly; lse is untouched."""
    q8, k8, v8, sq, sk, sv = _codes_problem(64, 200, 32, 31)
    o1, l1 = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, False)
    o2, l2 = F.attention_fp8(q8, k8, v8, sq, sk, sv * 2, 0.3, False)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(l1, l2)


def test_fp8_causal_first_row():
    q8, k8, v8, sq, sk, sv = _codes_problem(10, 10, 16, 41)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, True)
    v0 = F.dequantize(v8, sv)[:, 0]
    np.testing.assert_allclose(o[:, 0], v0, rtol=2.0 ** -4, atol=1e-12)
    s00 = 0.3 * np.sum(F.dequantize(q8, sq)[:, 0] * F.dequantize(k8, sk)[:, 0], axis=-1)
    np.testing.assert_allclose(lse[:, 0], s00, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_rows_option(causal):
    q8, k8, v8, sq, sk, sv = _codes_problem(300, 260, 32, 61)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal)
    rows = [0, 5, 127, 128, 299]
    o_r, lse_r = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal, rows=rows)
    np.testing.assert_allclose(o_r, o[:, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse_r, lse[:, rows], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ambiguity_bound_covers_perturbation(causal):
    """Nudging every score by ~1e-6 relative (as fp32 arithmetic does) moves O
    by no more than the ambiguity bound plus the smooth change of the weights."""
    q8, k8, v8, sq, sk, sv = _codes_problem(120, 333, 32, 71)
    sq = sq * 100  # sharper softmax: larger weights, so flips matter
    # a relative nudge eps of the scores moves each pre-rounding weight by
    # ln(2) |t| eps relative; |t| < 14 here, so ambiguity 1e-3 covers eps = 1e-4
    t = np.abs(F.dequantize(q8, sq) @ np.swapaxes(F.dequantize(k8, sk), -1, -2)) * 0.3 * F.LOG2E
    assert 5 < t.max() < 14
    o, lse, flip = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal, ambiguity=1e-3)
    assert np.all(flip >= 0)
    o2, _ = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3 * (1 + 1e-4), causal)
    # besides flips, the nudge moves l (and the unrounded weights) by ~1e-3 relative
    moved = np.abs(o2 - o) - 2e-3 * np.abs(o)
    assert np.all(moved <= flip + 1e-12), moved.max()
    assert np.any(np.abs(o2 - o) > 2e-3 * np.abs(o) + 1e-12)  # some code did flip
    o0 = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal)
    assert len(o0) == 2 and np.array_equal(o0[0], o)


def test_fp8_empty_keys():
    q8, k8, v8, sq, sk, sv = _codes_problem(5, 0, 16, 51)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk[:, :0], sv[:, :0], 0.3, False)
    assert np.all(o == 0) and np.all(lse == -np.inf)


# ------------------------------------------------------------------ method-level claim

def _fp8_rmse(w, q, k, v, signs, per_tensor, nq_sample):
    qs, ks = (signs, signs) if not per_tensor else (None, None)
    q8, sq = F.quantize(q, qs, per_tensor)
    k8, sk = F.quantize(k, ks, per_tensor)
    v8, sv = F.quantize(v, None, per_tensor)
    o, _ = F.attention_fp8(q8[..., :nq_sample, :], k8, v8, sq[..., :(nq_sample + 127) // 128], sk, sv, w.scale)
    truth, _ = oracle.attention(q[..., :nq_sample, :], k, v, w.scale)
    return F.rmse(o, truth)


@pytest.mark.slow
def test_incoherent_block_beats_per_tensor_on_outliers():
    """Same distribution as the fp8 outlier workload, one head, 256 queries x 8192 keys."""
    w = W.Workload("fp8_outlier_sample", 1, 1, 8192, 8192, 128, "fp8", False, seed=0, outliers=4)
    inp = W.make_inputs(w)
    e_blk = _fp8_rmse(w, inp["q"], inp["k"], inp["v"], inp["signs"], False, 256)
    e_pt = _fp8_rmse(w, inp["q"], inp["k"], inp["v"], inp["signs"], True, 256)
    assert e_pt / e_blk >= 2.0, (e_pt, e_blk)


@pytest.mark.slow
def test_fp8_rmse_normal_inputs():
    w = W.Workload("fp8_normal_sample", 1, 1, 8192, 8192, 128, "fp8", False, seed=0)
    inp = W.make_inputs(w)
    e_blk = _fp8_rmse(w, inp["q"], inp["k"], inp["v"], inp["signs"], False, 256)
    assert e_blk <= 3e-2


# ------------------------------------------------------------------ planted mistakes

def test_mutation_unnormalised_rotation(monkeypatch):
    monkeypatch.setattr(F, "rotation_matrix", lambda s: np.asarray(s)[:, None] * F.sylvester(len(s)))
    with pytest.raises(AssertionError):
        test_rotation_preserves_scores(64)


def test_mutation_ties_away(monkeypatch):
    orig = np.rint
    monkeypatch.setattr(F.np, "rint", lambda a: np.floor(a + 0.5) if np.ndim(a) else orig(a))
    try:
        with pytest.raises(AssertionError):
            test_round_matches_torch_cast_sweep()
    finally:
        monkeypatch.undo()


def test_mutation_wrong_fp8_max(monkeypatch):
    monkeypatch.setattr(F, "E4M3_MAX", 240.0)
    with pytest.raises(AssertionError):
        test_quantize_properties(False, True)


# ------------------------------------------------------------------ variable-length batches

VARLEN_LENS = [130, 1, 0, 256, 300, 127]  # ragged, a one-token and an empty sequence


def _packed(lens, d, seed):
    cu = W.cu_seqlens(lens)
    x = np.random.default_rng(seed).standard_normal((3, int(cu[-1]), d)).astype(np.float32)
    x *= np.exp(np.random.default_rng(seed + 1).uniform(-3, 3, (3, int(cu[-1]), 1))).astype(np.float32)
    return x, cu


def _owned_entries(lens, tile=128):
    """Scale entry of every (sequence, tile), brute force from the layout."""
    offs = F.varlen_tile_offsets(W.cu_seqlens(lens), tile)
    return [int(offs[b]) + t for b, n in enumerate(lens) for t in range((n + tile - 1) // tile)]


def test_varlen_tile_layout():
    cu = W.cu_seqlens(VARLEN_LENS)
    # cu = 0, 130, 131, 131, 387, 687: floor(cu / 128) + b = 0, 2, 3, 4, 7, 10;
    # tiles per sequence 2, 1, 0, 2, 3, 1 -> entries 0 1 | 2 | - | 4 5 | 7 8 9 | 10
    assert F.varlen_tile_offsets(cu).tolist() == [0, 2, 3, 4, 7, 10]
    assert _owned_entries(VARLEN_LENS) == [0, 1, 2, 4, 5, 7, 8, 9, 10]
    assert F.varlen_scale_len(int(cu[-1]), len(VARLEN_LENS)) == (814 + 127) // 128 + 6


def test_varlen_tile_layout_disjoint_and_bounded():
    """Every (sequence, tile) gets its own entry, below varlen_scale_len, for
    random length mixes with empty, one-token and tile-aligned sequences."""
    rng = np.random.default_rng(3)
    for _ in range(300):
        nseq = int(rng.integers(1, 40))
        lens = [int(x) for x in rng.choice([0, 1, 127, 128, 129, 256, int(rng.integers(0, 2000))], nseq)]
        for tile in (64, 128):
            ent = _owned_entries(lens, tile)
            assert len(set(ent)) == len(ent)
            assert all(0 <= e < F.varlen_scale_len(sum(lens), nseq, tile) for e in ent)
            assert ent == sorted(ent)


@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_varlen_tiles_restart_per_sequence(rotate):
    """Each sequence's tiles start at its first token: the largest magnitude
    of every (head, sequence tile) lands on 448 and the codes round to
    nearest, checked per sequence with the dense property checker; entries
    that no tile owns stay 1."""
    d = 64
    x, cu = _packed(VARLEN_LENS, d, 5)
    s = RNG.choice([-1.0, 1.0], d).astype(np.float32) if rotate else None
    codes, scales = F.quantize_varlen(x, cu, s)
    assert codes.shape == x.shape and scales.shape == (3, F.varlen_scale_len(x.shape[1], len(VARLEN_LENS)))
    offs = F.varlen_tile_offsets(cu)
    x_rot = F.rotate(x, s) if rotate else x.astype(np.float64)
    for b in range(len(VARLEN_LENS)):
        a, e = int(cu[b]), int(cu[b + 1])
        if e > a:
            nt = (e - a + 127) // 128
            _check_quantized(x_rot[:, a:e], codes[:, a:e], scales[:, offs[b]:offs[b] + nt], 128, False)
    free = np.ones(scales.shape[-1], bool)
    free[_owned_entries(VARLEN_LENS)] = False
    assert np.all(scales[:, free] == 1.0)


def test_quantize_varlen_aligned_equals_dense():
    """Sequences whose lengths are multiples of 128 tile the packed tensor
    exactly as the dense layout does, so codes and scales coincide with
    `quantize` of the whole tensor as one batch entry."""
    x, cu = _packed([256, 128, 384], 64, 9)
    codes, scales = F.quantize_varlen(x, cu)
    ref_c, ref_s = F.quantize(x[None])
    assert np.array_equal(codes, ref_c[0])
    assert _owned_entries([256, 128, 384]) == [0, 1, 3, 5, 6, 7]
    assert np.array_equal(scales[:, [0, 1, 3, 5, 6, 7]], ref_s[0])


def test_quantize_varlen_per_tensor_equals_dense():
    x, cu = _packed(VARLEN_LENS, 64, 13)
    codes, scales = F.quantize_varlen(x, cu, per_tensor=True)
    ref_c, ref_s = F.quantize(x[None], per_tensor=True)
    assert np.array_equal(codes, ref_c[0])
    assert np.all(scales == ref_s.flat[0])


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_varlen_reduces_to_exact_varlen(causal):
    """With P unrounded the fp8 emulation of a packed batch equals the exact
    variable-length definition on the dequantised inputs (each sequence with
    its own scale tiles; a different code path: exact.attention_varlen)."""
    d = 32
    lens_q, lens_k = [130, 1, 0, 200], [130, 5, 3, 129]
    cq, ck = W.cu_seqlens(lens_q), W.cu_seqlens(lens_k)
    nq, nk = int(cq[-1]), int(ck[-1])
    q8 = W.random_e4m3_codes((2, nq, d), 21, max_exp_field=9)
    k8 = W.random_e4m3_codes((2, nk, d), 22, max_exp_field=9)
    v8 = W.random_e4m3_codes((2, nk, d), 23, max_exp_field=9)
    sq = W.random_scales((2, F.varlen_scale_len(nq, 4)), 24)
    sk = W.random_scales((2, F.varlen_scale_len(nk, 4)), 25)
    sv = W.random_scales((2, F.varlen_scale_len(nk, 4)), 26)
    o, lse = F.attention_fp8_varlen(q8, k8, v8, sq, sk, sv, cq, ck, 0.3, causal, quantize_p=False)

    def deq(codes, scales, cu):  # dequantise each sequence with its own tiles
        out = np.zeros(codes.shape)
        offs = F.varlen_tile_offsets(cu)
        for b in range(len(cu) - 1):
            a, e = int(cu[b]), int(cu[b + 1])
            vals = F.e4m3_decode(codes[:, a:e])
            rows = offs[b] + np.arange(e - a) // 128
            out[:, a:e] = vals * scales[:, rows].astype(np.float64)[..., None]
        return out

    ref_o, ref_l = oracle.attention_varlen(deq(q8, sq, cq), deq(k8, sk, ck), deq(v8, sv, ck), cq, ck, 0.3, causal)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], ref_l[fin], rtol=1e-13, atol=1e-12)


def test_fp8_varlen_single_sequence_equals_dense():
    q8, k8, v8, sq, sk, sv = _codes_problem(300, 300, 32, 31)
    cu = np.array([0, 300])
    pad = lambda s: np.concatenate([s, np.ones((2, 1), np.float32)], axis=-1)  # noqa: E731
    o, lse = F.attention_fp8_varlen(q8, k8, v8, pad(sq), pad(sk), pad(sv), cu, cu, 0.3, True)
    ref_o, ref_l = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, True)
    assert np.array_equal(o, ref_o) and np.array_equal(lse, ref_l)


# ------------------------------------------------------------------ P-code scale and V scales

def _two_key_row(t1: float):
    """One query, two keys in one 128-key tile, scales 1: key 0 scores t = 0
    (so M = 0 and its weight is 1), key 1 scores t1 (base 2).  V: key 0 is
    the zero row, key 1 the all-ones row, so O = (code of key 1) 2^-8 / l in
    every column."""
    d = 16
    one, sixteen = F.e4m3_encode(1.0), F.e4m3_encode(16.0)
    q8 = np.zeros((1, d), np.uint8)
    q8[0, 0] = one
    k8 = np.zeros((2, d), np.uint8)
    k8[1, 0] = F.e4m3_encode(-16.0)
    v8 = np.zeros((2, d), np.uint8)
    v8[1, :] = one
    ones = np.ones(1, np.float32)
    scale = -t1 / (16.0 * F.LOG2E)  # t(key 1) = scale * (-16) * log2(e) = t1
    assert sixteen != 0
    return q8, k8, v8, ones, ones, ones, scale


@pytest.mark.parametrize("t1,code", [(-17.4, 2.0 ** -9), (-17.9, 2.0 ** -9), (-16.4, 2.0 ** -8),
                                     (-18.2, 0.0), (-12.0, 2.0 ** -4)])
def test_p_scale_smallest_weights(t1, code):
    """The P codes are e4m3(2^8 p): a weight p = 2^t1 lands on the code of
    2^(t1 + 8), so the smallest subnormal code 2^-9 holds weights from just
    above 2^-18 (the tie at 2^-18 rounds to 0) up to 1.5 * 2^-17, and O of
    the two-key row is that code times 2^-8 over l = 1 + 2^t1 (closed form)."""
    q8, k8, v8, sq, sk, sv, scale = _two_key_row(t1)
    r = F.attention_fp8(q8, k8, v8, sq, sk, sv, scale, parts=True)
    assert r["M"][0] == 0.0 and r["p8"][0, 0] == 256.0
    assert r["p8"][0, 1] == code
    expect = code * 2.0 ** -8 / (1.0 + 2.0 ** t1)
    np.testing.assert_allclose(r["o"][0], np.full(16, expect), rtol=1e-12, atol=0)
    np.testing.assert_allclose(r["lse"][0], np.log1p(2.0 ** t1), rtol=0, atol=1e-12)


def test_p_scale_largest_code():
    """scale = 0: every weight is 1 (M = 0), so the keys of the tile with the
    largest V scale code to 2^8 = 256 exactly and those of a tile whose V
    scale is half of it to 128 (w = 1/2 folded into P)."""
    q8, k8, v8, sq, sk, sv = _codes_problem(3, 256, 16, 81)
    sv = np.array([[0.25, 0.5], [0.5, 0.25]], np.float32)
    r = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.0, parts=True)
    assert np.all(r["p8"][0, :, :128] == 128.0) and np.all(r["p8"][0, :, 128:] == 256.0)
    assert np.all(r["p8"][1, :, :128] == 256.0) and np.all(r["p8"][1, :, 128:] == 128.0)
    ref = F.dequantize(v8, sv).mean(axis=-2)  # every code exact: O is the mean of V
    np.testing.assert_allclose(r["o"], np.broadcast_to(ref[:, None, :], r["o"].shape), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("log2_scale", [7, 9])
def test_mutation_p_scale(monkeypatch, log2_scale):
    """A P scale of 2^7 drops the weights between 2^-18 and 2^-17 (and a
    2^-17.4 weight codes to 0); 2^9 codes the largest weights to 448
    (saturation) and moves the small ones up a code: each pin catches both."""
    monkeypatch.setattr(F, "P_SCALE_LOG2", log2_scale)
    with pytest.raises(AssertionError):
        test_p_scale_smallest_weights(-17.4, 2.0 ** -9)
    with pytest.raises(AssertionError):
        test_p_scale_largest_code()


@pytest.mark.parametrize("causal", [False, True])
def test_zero_v_scale_tile(causal):
    """A V tile whose scale is 0 (the caller's scales may be 0): its keys
    still count in the softmax sum l, and they add nothing to O.  Against
    plain attention on the dequantised inputs (that tile's V rows are 0),
    exact with P unrounded and within the P-rounding bound with it."""
    q8, k8, v8, sq, sk, sv = _codes_problem(150, 300, 32, 91)
    sv = sv.copy()
    sv[0, 1] = 0.0
    qd, kd, vd = F.dequantize(q8, sq), F.dequantize(k8, sk), F.dequantize(v8, sv)
    assert np.all(vd[0, 128:256] == 0)
    ref_o, ref_l = oracle.attention(qd, kd, vd, 0.3, causal)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal, quantize_p=False)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13, atol=1e-12)
    o8, lse8 = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal)
    np.testing.assert_allclose(lse8, ref_l, rtol=1e-13, atol=1e-12)
    p, _, _ = oracle.softmax_rows(oracle.scores(qd, kd, 0.3, causal))
    bound = (2.0 ** -4 * p + 2.0 ** -18) @ np.abs(vd) * 1.000001
    assert np.all(np.abs(o8 - ref_o) <= bound + 1e-12)


def test_all_zero_v_scales():
    q8, k8, v8, sq, sk, _ = _codes_problem(20, 130, 16, 93)
    sv = np.zeros((2, 2), np.float32)
    o, lse = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, False)
    _, ref_l = oracle.attention(F.dequantize(q8, sq), F.dequantize(k8, sk), np.zeros((2, 130, 16)), 0.3)
    assert np.all(o == 0) and not np.any(np.isnan(o))
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13, atol=1e-12)


def test_rowmax_reading():
    """The other plain reading of the P rounding (V scale applied per tile
    after the product): unrounded, both readings are plain attention on the
    dequantised inputs; with equal V scales (w = 1) they round identically;
    with unequal scales they differ."""
    q8, k8, v8, sq, sk, sv = _codes_problem(90, 300, 32, 95)
    a = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, quantize_p=False, p_mode="rowmax")
    b = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, quantize_p=False)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)
    eq = np.full_like(sv, 0.125)
    a = F.attention_fp8(q8, k8, v8, sq, sk, eq, 0.3, p_mode="rowmax")
    b = F.attention_fp8(q8, k8, v8, sq, sk, eq, 0.3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    a = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, p_mode="rowmax")
    b = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3)
    assert not np.allclose(a[0], b[0], rtol=0, atol=1e-9)


def test_quantize_tiny_amax():
    """amax below 448 * 2^-149: amax / 448 underflows fp32, so the scale is
    the smallest positive fp32 2^-149, and each code is x / 2^-149, an
    integer (x is a multiple of 2^-149) rounded to e4m3."""
    x = np.zeros((1, 1, 128, 64), np.float32)
    vals = np.array([1, 3, 17, 100, 300], np.float64)
    x[0, 0, 0, :5] = (vals * 2.0 ** -149).astype(np.float32)
    x[0, 0, 1, :5] = -x[0, 0, 0, :5]
    assert np.array_equal(x[0, 0, 0, :5].astype(np.float64) * 2.0 ** 149, vals)
    codes, scales = F.quantize(x)
    assert scales[0, 0, 0] == np.float32(2.0 ** -149)
    got = F.e4m3_decode(codes[0, 0, :2, :5])
    expect = F.e4m3_round(vals)  # 17 -> 16, 100 -> 96, 300 -> 288
    assert np.array_equal(got[0], expect) and np.array_equal(got[1], -expect)
    assert list(expect) == [1.0, 3.0, 16.0, 96.0, 288.0]


def test_p_rounding_follows_the_running_max():
    """P is rounded tile by tile against the running integer max, the order
    of the blog's online-softmax recurrence (§2.2: block j's term enters as
    exp(S_j - m_new) V_j).  One query; 256 keys in two 128-key tiles with V
    scales 1: tile 0 holds t = 0 (key 0) and t = -17.4 (key 1), tile 1 holds
    t = 9.7875 (key 128); every other key scores -487 (weight 0).  Running
    max: M_0 = 0, then M_1 = M = 10.  V rows one-hot (key 0 -> column 0,
    key 1 -> 1, key 128 -> 2), so column c of O is the effective code of its
    key times 2^-8 / l:
      key 0:   e4m3(2^8) 2^(0 - 10)        = 2^-2
      key 1:   e4m3(2^-9.4) 2^-10 = 2^-9 2^-10  (rounded against M = 10 it
               would be e4m3(2^-19.4) = 0)
      key 128: e4m3(2^7.7875) = 224
    with l = 2^-10 + 2^-27.4 + 2^-0.2125."""
    d = 16
    q8 = np.zeros((1, d), np.uint8)
    q8[0, 0] = F.e4m3_encode(1.0)
    k8 = np.zeros((256, d), np.uint8)
    kv = np.full(256, -448.0)
    kv[0], kv[1], kv[128] = 0.0, -16.0, 9.0
    k8[:, 0] = F.e4m3_encode(kv)
    v8 = np.zeros((256, d), np.uint8)
    v8[0, 0] = v8[1, 1] = v8[128, 2] = F.e4m3_encode(1.0)
    ones = np.ones(2, np.float32)
    scale = 17.4 / (16.0 * F.LOG2E)  # t(key 1) = -17.4, t(key 128) = 17.4 * 9 / 16 = 9.7875
    r = F.attention_fp8(q8, k8, v8, ones[:1], ones, ones, scale, parts=True)
    assert r["M"][0] == 10.0 and list(r["M_tile"][0]) == [0.0, 10.0]
    l = 2.0 ** -10 + 2.0 ** (-17.4 - 10) + 2.0 ** (9.7875 - 10)
    np.testing.assert_allclose(r["l"][0], l, rtol=1e-12)
    expect = np.array([2.0 ** -2, 2.0 ** -19, 224.0]) * 2.0 ** -8 / l
    np.testing.assert_allclose(r["o"][0, :3], expect, rtol=1e-12, atol=0)
    assert np.all(r["o"][0, 3:] == 0)
    np.testing.assert_allclose(r["lse"][0], (10 + np.log2(l)) / F.LOG2E, rtol=0, atol=1e-12)


def test_p_rounding_running_max_per_key_block():
    """With 64-key blocks (the d = 256 kernel's tiling) the running max rises
    within a 128-key scale tile.  One query; keys 0 (t = 0) and 1 (t = -17.4)
    in block 0, key 64 (t = 9.7875) in block 1 of the same scale tile, every
    other key at weight 0; V rows one-hot.  Blocks of 64: M_0 = 0, so key 1
    codes as e4m3(2^-9.4) = 2^-9 against M_0 and enters O as 2^-19 (in units
    of M = 10); blocks of 128: M_0 = 10 already, and key 1's code is
    e4m3(2^-19.4) = 0.  Without P rounding the two agree exactly."""
    d = 16
    q8 = np.zeros((1, d), np.uint8)
    q8[0, 0] = F.e4m3_encode(1.0)
    k8 = np.zeros((128, d), np.uint8)
    kv = np.full(128, -448.0)
    kv[0], kv[1], kv[64] = 0.0, -16.0, 9.0
    k8[:, 0] = F.e4m3_encode(kv)
    v8 = np.zeros((128, d), np.uint8)
    v8[0, 0] = v8[1, 1] = v8[64, 2] = F.e4m3_encode(1.0)
    one = np.ones(1, np.float32)
    scale = 17.4 / (16.0 * F.LOG2E)
    r64 = F.attention_fp8(q8, k8, v8, one, one, one, scale, parts=True, block=64)
    r128 = F.attention_fp8(q8, k8, v8, one, one, one, scale, parts=True)
    assert list(r64["M_tile"][0]) == [0.0, 10.0] and list(r128["M_tile"][0]) == [10.0]
    l = 2.0 ** -10 + 2.0 ** (-17.4 - 10) + 2.0 ** (9.7875 - 10)
    np.testing.assert_allclose(r64["o"][0, :3], np.array([2.0 ** -2, 2.0 ** -19, 224.0]) * 2.0 ** -8 / l,
                               rtol=1e-12, atol=0)
    np.testing.assert_allclose(r128["o"][0, :3], np.array([2.0 ** -2, 0.0, 224.0]) * 2.0 ** -8 / l,
                               rtol=1e-12, atol=0)
    e64 = F.attention_fp8(q8, k8, v8, one, one, one, scale, quantize_p=False, block=64)
    e128 = F.attention_fp8(q8, k8, v8, one, one, one, scale, quantize_p=False)
    np.testing.assert_allclose(e64[0], e128[0], rtol=1e-14)
    with pytest.raises(ValueError):
        F.attention_fp8(q8, k8, v8, one, one, one, scale, block=48)


# ------------------------------------------------------------- key chunks

def _split_problem(lead, nq, nk, d, seed):
    q8 = W.random_e4m3_codes(lead + (nq, d), seed, max_exp_field=9)
    k8 = W.random_e4m3_codes(lead + (nk, d), seed + 1, max_exp_field=9)
    v8 = W.random_e4m3_codes(lead + (nk, d), seed + 2, max_exp_field=9)
    sq = W.random_scales(lead + ((nq + 127) // 128,), seed + 3)
    sk = W.random_scales(lead + ((nk + 127) // 128,), seed + 4)
    sv = W.random_scales(lead + ((nk + 127) // 128,), seed + 5)
    return q8, k8, v8, sq, sk, sv


def test_fp8_split_bounds_whole_scale_tiles():
    for nk in (0, 1, 127, 128, 129, 700, 1000, 4096):
        for s in (1, 2, 3, 7, 40):
            b = F.split_bounds_fp8(nk, s)
            assert len(b) == s and b[0][0] == 0 and b[-1][1] == nk
            assert all(e0 == b1 for (_, e0), (b1, _) in zip(b[:-1], b[1:]))
            assert all(kb % 128 == 0 for kb, ke in b if ke > kb)  # empty chunks sit at nk
    assert F.split_bounds_fp8(700, 3) == [(0, 256), (256, 512), (512, 700)]


@pytest.mark.parametrize("causal", [False, True])
def pin_fp8_split_unrounded_equals_exact(causal, split=F.attention_fp8_splitkv):
    """With P unrounded the merged chunks equal the exact attention of the
    dequantised operands (a different code path, oracle.attention): chunk
    bounds, the scale tiles each chunk reads, the absolute causal indices
    and the merge all have to be right.  Rows whose whole chunk lies above
    the diagonal contribute nothing."""
    q8, k8, v8, sq, sk, sv = _split_problem((2,), 300, 700, 32, 41)
    for S in (1, 3, 6):
        o, lse = split(q8, k8, v8, sq, sk, sv, 0.25, causal, num_splits=S, quantize_p=False)
        ref_o, ref_l = oracle.attention(F.dequantize(q8, sq), F.dequantize(k8, sk), F.dequantize(v8, sv), 0.25, causal)
        np.testing.assert_allclose(o, ref_o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, ref_l, rtol=1e-12, atol=1e-12)


test_fp8_split_unrounded_equals_exact = pin_fp8_split_unrounded_equals_exact


def test_fp8_split_one_chunk_is_the_dense_emulation():
    q8, k8, v8, sq, sk, sv = _split_problem((2,), 200, 300, 32, 43)
    for causal in (False, True):
        o, lse = F.attention_fp8_splitkv(q8, k8, v8, sq, sk, sv, 0.3, causal, num_splits=1)
        ref_o, ref_l = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.3, causal)
        assert np.allclose(o, ref_o, rtol=1e-14, atol=1e-15) and np.array_equal(np.isneginf(lse), np.isneginf(ref_l))
        np.testing.assert_allclose(lse[np.isfinite(ref_l)], ref_l[np.isfinite(ref_l)], rtol=1e-14)


def test_fp8_split_rounded_within_bound():
    """P rounded per chunk: the merged result stays within what rounding P to
    three mantissa bits can do against the unrounded split (relative RMSE
    below 2^-4)."""
    q8, k8, v8, sq, sk, sv = _split_problem((2,), 128, 1000, 64, 47)
    a, _ = F.attention_fp8_splitkv(q8, k8, v8, sq, sk, sv, 0.125, False, num_splits=4)
    b, _ = F.attention_fp8_splitkv(q8, k8, v8, sq, sk, sv, 0.125, False, num_splits=4, quantize_p=False)
    rel = np.sqrt(np.mean((a - b) ** 2)) / np.sqrt(np.mean(b ** 2))
    assert 0 < rel < 2.0 ** -4


def test_mutation_split_chunk_offset(monkeypatch):
    """A chunk whose causal mask used local key indices: the pin fails."""
    orig = F.attention_fp8

    def mutant(*a, **kw):
        kw["k_offset"] = 0
        return orig(*a, **kw)

    monkeypatch.setattr(F, "attention_fp8", mutant)
    with pytest.raises(AssertionError):
        pin_fp8_split_unrounded_equals_exact(True)
