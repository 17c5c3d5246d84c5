"""GPU parity of the fp8 path: pre-processing (rotation + block quantisation)
and the e4m3 attention kernel, against the fp64 oracle.

* Pre-processing without rotation takes every decision on the same fp32
  values as the oracle (x, amax, s = amax/448 and x/s are all exact or
  correctly rounded), so codes and scales must be bit-identical.  With the
  rotation the device sums the Hadamard butterflies in fp32 while the oracle
  rotates in fp64; scales then agree to a few ulps and a code may differ by
  one step only where the oracle's value sits next to a rounding midpoint.
* The attention kernel is fed e4m3 codes and scales drawn by the input
  generator (no quantisation arithmetic), and compared with the oracle's
  fp8 emulation (same P rounding).  The gfx950 e4m3 MFMA adds its products
  in groups of 8 consecutive k-indices, truncating each toward zero 13 bits
  below the exponent of the group's largest product (a property of the
  instruction, measured with a probe), so it is not an exact fp32 dot
  product.  The codes are drawn from {+-1, +-1.5, +-2, +-3,
  +-4} with power-of-two scales, for which the S = K Q^T products are added
  exactly; the PV product's truncation is bounded from the oracle's P codes.
  Bar: max |O - O_emu| <= 4e-3 (the bf16 output rounding, half an ulp of
  |O| < 0.5 <= 2^-10, plus fp32 accumulation) + that bound + the flips
  below; lse within 1e-3 relative.  A P code is not unique where its
  pre-rounding value lies within fp32 error (3e-5 relative: the fp32
  score and the exp2) of an e4m3 midpoint: there either neighbour is valid,
  so the bar of each element grows by the oracle's bound on what
  re-rounding all such codes can change.
* End to end at the full fp8 shape (B=2 H=16 N=8192 d=128), over the whole
  output: RMSE against the fp64 truth <= 3e-2 on N(0,1) inputs; with outlier
  channels, the per-tensor RMSE is >= 2x the block + Hadamard RMSE; and on
  sampled rows of four heads the device RMSE is within 10 % of the
  emulation's.
* Codes from the quantiser (N(0,1) and outlier inputs, codes up to 448,
  subnormals, arbitrary fp32 scales): element-wise against the emulation,
  with an allowance derived from the MFMA's accumulation (the query rows
  carry one nonzero channel per accumulation group, so S is rounded only in
  fp32; the PV products' truncation is bounded) and from the code flips,
  l and M it can cause.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import exact as OX
from oracle import fp8 as F
import workloads as W
from gpu_util import sample_rows

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# ---------------------------------------------------------------- pre-processing

@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_prep_no_rotation_bitwise(gpu_lib, in_dtype, d, per_tensor):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((2, 3, 300, d), dtype=np.float32) * np.float32(3.0)
    x[1, 1, 128:256] = 0.0  # an all-zero tile: scale 1, codes 0
    xt = torch.from_numpy(x) if in_dtype == "f32" else W.to_dtype(x, in_dtype)
    codes, scales = gpu_lib.fp8_quantize(xt.cuda(), None, per_tensor)
    torch.cuda.synchronize()
    ref_codes, ref_scales = F.quantize(xt.double().numpy().astype(np.float32), None, per_tensor)
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != ref_codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("magnitude", [1e-32, 1e-20, 3e4])
def test_prep_scale_range_bitwise(gpu_lib, magnitude):
    """Tiles whose scale is tiny (the kernel then divides with the IEEE
    quotient instead of the reciprocal-and-correction form) or large: codes
    and scales still equal the oracle's fp32 decisions bit for bit."""
    rng = np.random.default_rng(abs(int(np.log10(magnitude))) + 7)
    x = (rng.standard_normal((1, 2, 256, 128), dtype=np.float32) * np.float32(magnitude)).astype(np.float32)
    x[0, 1, 128:] *= np.float32(1e-3)  # a second, smaller tile scale
    codes, scales = gpu_lib.fp8_quantize(_dev(x), None)
    torch.cuda.synchronize()
    ref_codes, ref_scales = F.quantize(x, None)
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    bad = np.argwhere(codes.cpu().numpy() != ref_codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("outliers", [0, 4])
def test_prep_rotation(gpu_lib, d, outliers):
    w = W.Workload("prep", 2, 3, 333, 333, d, "fp8", False, seed=d + outliers, outliers=outliers)
    inp = W.make_inputs(w)
    x, signs = inp["q"], inp["signs"]
    codes, scales = gpu_lib.fp8_quantize(_dev(x), _dev(signs))
    torch.cuda.synchronize()
    ref_codes, ref_scales = F.quantize(x, signs)
    s_gpu = scales.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(s_gpu, ref_scales, rtol=4 * 2.0 ** -23, atol=0)
    got = codes.cpu().numpy()
    diff = got != ref_codes
    assert diff.mean() <= 1e-3, f"{diff.sum()} of {diff.size} codes differ"
    if diff.any():
        # every difference is one step between neighbours, at a rounding midpoint
        g = F.e4m3_decode(got[diff])
        o = F.e4m3_decode(ref_codes[diff])
        xr = F.rotate(x, signs)
        n = x.shape[-2]
        rs = np.repeat(ref_scales.astype(np.float64), 128, axis=-1)[..., :n][..., None]
        y = (xr / rs)[diff]
        mid = (g + o) / 2
        # fp32 butterflies: each of the log2(d) stages and the final scaling
        # rounds by at most 2^-24 of a partial sum bounded by sum_i |x_i|
        row_l1 = np.broadcast_to(np.abs(x).sum(-1, keepdims=True) / np.sqrt(d), x.shape)[diff]
        bound = (np.log2(d) + 3) * 2.0 ** -24 * row_l1 / np.broadcast_to(rs, x.shape)[diff]
        assert np.all(np.abs(y - mid) <= bound + 1e-12), "a code differs away from a midpoint"
        grid = np.unique(F.e4m3_decode(np.arange(256, dtype=np.uint8))[:127])
        gi, oi = np.searchsorted(grid, np.abs(g)), np.searchsorted(grid, np.abs(o))
        assert np.all(np.abs(gi - oi) == 1) and np.all(np.sign(g) == np.sign(o))


# ---------------------------------------------------------------- attention kernel

# +-1, +-1.5, +-2, +-3, +-4: products are multiples of 1/4 below 16, which the
# 8-product groups of the e4m3 MFMA (truncated 13 bits below the group's
# largest product) add exactly, so S has no hardware rounding.
EXACT_CODES = [0x38, 0x3C, 0x40, 0x44, 0x48, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8]


# key-block length of the kernel's running max per head dimension (the
# emulation's ``block``): 128-key tiles, 64 at d = 256
BLOCK = {64: 128, 128: 128, 256: 64}


def _exact_problem(B, H, nq, nk, seed, d=128):
    nt = lambda n: (n + 127) // 128  # noqa: E731
    q8 = W.random_codes_from(EXACT_CODES, (B, H, nq, d), seed)
    k8 = W.random_codes_from(EXACT_CODES, (B, H, nk, d), seed + 1)
    v8 = W.random_codes_from(EXACT_CODES, (B, H, nk, d), seed + 2)
    sq = W.random_pow2_scales((B, H, nt(nq)), seed + 3, -1, 0)
    sk = W.random_pow2_scales((B, H, nt(nk)), seed + 4, -1, 0)
    sv = W.random_pow2_scales((B, H, nt(nk)), seed + 5, -7, -4)
    return q8, k8, v8, sq, sk, sv


# The e4m3 MFMA (v_mfma_f32_32x32x64_f8f6f4) adds its products in groups of
# MFMA_GROUP consecutive k-indices, truncating each product toward zero at
# 2^(e - MFMA_KEEP_BITS), e the exponent of the group's largest product; the
# group sums then add without further loss at these magnitudes (measured
# with a probe: 256 + 1.25 * 2^-4 -> 256.0625, 256 + 2^-6 -> 256, two 448s
# and 62 products of 2^-9 -> 896 + 56 * 2^-9).
MFMA_GROUP = 8
MFMA_KEEP_BITS = 13


def _pv_bound(parts):
    """Bound on the PV product's truncation inside the e4m3 MFMA, in O units.

    In the kernel's PV operands the k-index 32 h + j of lane half h holds key
    64 g + 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4, so each group of 8
    k-indices holds keys of one aligned 16-key block.  Per block, every
    product other than its group's largest loses less than 2^(e - 13), e the
    exponent of the block's largest |P8 v8| (taken with the key's largest |v8|
    over the columns).  Scaled like O: max s_v 2^-8 / l.
    """
    p8, vc, l, svm = parts["p8"], parts["v_codes"], parts["l"], parts["sv_max"]
    vmax = np.abs(vc).max(-1)  # [..., Nk]
    prod = p8 * vmax[..., None, :]  # [..., Nq, Nk]
    nk = prod.shape[-1]
    tot = np.zeros(prod.shape[:-1])
    for j0 in range(0, nk, 16):
        blk = prod[..., j0:j0 + 16]
        m = blk.max(-1)
        cnt = np.count_nonzero(blk, axis=-1)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        tot += np.where(cnt > 1, (cnt - 1) * np.exp2(e - MFMA_KEEP_BITS), 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(l > 0, tot * svm[..., None] / 256.0 / np.where(l > 0, l, 1.0), 0.0)
    return out[..., None]


def _s_bound(q8, k8):
    """Bound on the S product's truncation inside the e4m3 MFMA, in raw units
    (before the scale and the tile scales), per (query, key).

    The S operands hold channels 64 ks + 32 h .. + 31 of k-step ks in lane
    half h, so a group is 8 consecutive channels; every product other than
    the group's largest loses less than 2^(e - 13), e the exponent of the
    group's largest |q k|.  Returns [..., Nq, Nk].
    """
    qv, kv = F.e4m3_decode(q8), F.e4m3_decode(k8)
    d = qv.shape[-1]
    tot = np.zeros(qv.shape[:-1] + (kv.shape[-2],))
    for g in range(d // MFMA_GROUP):
        sl = slice(g * MFMA_GROUP, (g + 1) * MFMA_GROUP)
        qs, kk = qv[..., sl], kv[..., sl]
        nz = np.flatnonzero(np.any(qs != 0, axis=tuple(range(qs.ndim - 1))))
        if nz.size < 2:
            continue  # at most one product: exact
        prod = np.abs(qs[..., :, None, nz] * kk[..., None, :, nz])  # [..., Nq, Nk, nnz]
        m = prod.max(-1)
        cnt = np.count_nonzero(prod, axis=-1)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        tot += np.where(cnt > 1, (cnt - 1) * np.exp2(e - MFMA_KEEP_BITS), 0.0)
    return tot


def _quantiser_allowance(q8, k8, v8, sq, sk, sv, scale, causal, tile=128, block=128):
    """Per-element allowance of the e4m3 kernel against the fp8 emulation
    when the S product rounds (``_s_bound``), in O units, and the bound on the
    lse difference.

    A score moved by dt (base 2) moves its P value x = 2^(t - M + 8) w by the
    relative amount delta = 2^dt - 1 (plus 3e-5 for the fp32 score and exp2):
    (a) a code whose x lies within delta of a rounding midpoint may take the
    other neighbour (the emulation's ``ambiguity`` bound with a per-element
    delta); (b) l, an fp32 sum of the unrounded p, moves by the p-weighted
    mean of delta (plus 1e-5 for its fp32 additions), and O = sum P8 v / l
    with it; (c) where the running max of a key tile lies within dt of an
    integer, the kernel's running M may be the neighbouring integer from
    there on: the codes are then formed at half (or twice) the emulation's
    values, which is exact for normal codes and moves a code below 2^-4 (in
    its tile's units) by less than 2^-7.  Returns (the emulation's parts,
    allowance [..., Nq, d], lse bound [..., Nq])."""
    ref = F.attention_fp8(q8, k8, v8, sq, sk, sv, scale, causal, parts=True, block=block)
    nq, nk = q8.shape[-2], k8.shape[-2]
    rs = lambda sc, n: np.repeat(np.asarray(sc, np.float64), tile, axis=-1)[..., :n]  # noqa: E731
    cs = abs(scale) * F.LOG2E * rs(sq, nq)[..., :, None] * rs(sk, nk)[..., None, :]
    t = ref["t"]
    fin = np.isfinite(t)
    dt = cs * _s_bound(q8, k8) + 4 * 2.0 ** -24 * np.abs(np.where(fin, t, 0.0))
    delta = np.where(fin, np.expm1(dt * np.log(2.0)) + 3e-5, 0.0)
    flip = F.attention_fp8(q8, k8, v8, sq, sk, sv, scale, causal, ambiguity=delta, parts=True, block=block)["flip"]
    M, l = ref["M"], ref["l"]
    p = np.where(fin, np.exp2(np.where(fin, t, 0.0) - M[..., None]), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        dl = np.where(l > 0, (p * delta).sum(-1) / np.where(l > 0, l, 1.0), 0.0) + 1e-5
    lchg = np.abs(ref["o"]) * (dl / (1.0 - dl))[..., None]
    # the running max of the key blocks (before its ceiling): where one lies
    # within dt of an integer, the kernel's running M may differ by one there
    nkt = (nk + block - 1) // block
    tpad = np.concatenate([np.where(fin, t, -np.inf), np.full(t.shape[:-1] + (nkt * block - nk,), -np.inf)], -1)
    run = np.maximum.accumulate(tpad.reshape(t.shape[:-1] + (nkt, block)).max(-1), axis=-1)
    dmax = dt.max(-1)
    with np.errstate(invalid="ignore"):
        near = np.any(np.abs(run - np.rint(run)) <= dmax[..., None], axis=-1)
    small = (ref["x"] < 2.0 ** -4) & fin
    with np.errstate(invalid="ignore", divide="ignore"):
        norm = np.where(l > 0, ref["sv_max"][..., None] * 2.0 ** -8 / np.where(l > 0, l, 1.0), 0.0)
    m_amb = np.matmul(small * 2.0 ** -7 * np.exp2(ref["shift"]), np.abs(ref["v_codes"])) * (norm * near)[..., None]
    lse_bound = np.log(2.0) * (dmax + dl)
    return ref, flip + lchg + m_amb + _pv_bound(ref), lse_bound


def _run_fp8(attn, q8, k8, v8, sq, sk, sv, scale, causal):
    o, lse = attn.forward(_dev(q8), _dev(k8), _dev(v8), causal=causal, scale=scale,
                          q_scale=_dev(sq), k_scale=_dev(sk), v_scale=_dev(sv))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def _check(o, lse, o_ref, l_ref, what, tol=4e-3, allow=0.0):
    assert not np.any(np.isnan(o)) and not np.any(np.isnan(lse)), what
    err = np.abs(o - o_ref) - allow
    i = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err[i] <= tol, f"{what}: |O - O_emu| - allowance = {err[i]:.3e} at {i}"
    assert np.array_equal(np.isneginf(lse), np.isneginf(l_ref)), what
    fin = ~np.isneginf(l_ref)
    rel = np.abs(lse[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))
    assert rel.size == 0 or rel.max() <= 1e-3, f"{what}: lse rel err {rel.max():.3e}"


FP8_SHAPES = [(1, 1), (100, 100), (128, 128), (129, 300), (300, 129), (1000, 1000), (513, 2000)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,nq,nk", [(128,) + s for s in FP8_SHAPES]
                         + [(d, nq, nk) for d in (64, 256) for nq, nk in ((1, 1), (129, 300), (300, 129), (513, 1000))])
def test_fp8_kernel_vs_emulation(gpu_lib, causal, d, nq, nk):
    q8, k8, v8, sq, sk, sv = _exact_problem(2, 2, nq, nk, seed=nq + 3 * nk + d, d=d)
    o, lse = _run_fp8(gpu_lib, q8, k8, v8, sq, sk, sv, 0.0884, causal)
    ref = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.0884, causal, ambiguity=3e-5, parts=True, block=BLOCK[d])
    allow = ref["flip"] + _pv_bound(ref)
    _check(o, lse, ref["o"], ref["lse"], f"fp8 d{d} causal{causal} {nq}x{nk}", allow=allow)
    # the allowances stay a small part of the signal
    assert np.mean(allow) <= 0.25 * np.mean(np.abs(ref["o"])) + 1e-6


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_kernel_uniform_closed_form(gpu_lib, causal, d):
    """scale = 0: every visible key weighs the same and P is exact (2^8 w with
    w a power of two), so O is the mean (causal: prefix mean) of the
    dequantised V rows, up to the bf16 rounding of O."""
    nq = nk = 700
    q8, k8, v8, sq, sk, sv = _exact_problem(2, 3, nq, nk, seed=33, d=d)
    o, lse = _run_fp8(gpu_lib, q8, k8, v8, sq, sk, sv, 0.0, causal)
    vd = F.dequantize(v8, sv)
    if causal:
        ref = np.cumsum(vd, axis=-2) / np.arange(1, nk + 1)[:, None]
        lref = np.broadcast_to(np.log(np.arange(1, nq + 1)), lse.shape)
    else:
        ref = np.broadcast_to(vd.mean(-2, keepdims=True), o.shape)
        lref = np.full(lse.shape, np.log(nk))
    assert np.all(np.abs(o - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-7)
    np.testing.assert_allclose(lse, lref, rtol=0, atol=1e-5)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_kernel_empty_keys(gpu_lib, d):
    q8, _, _, sq, _, _ = _exact_problem(1, 2, 50, 1, seed=5, d=d)
    z8 = torch.zeros((1, 2, 0, d), dtype=torch.uint8, device="cuda")
    zs = torch.zeros((1, 2, 0), dtype=torch.float32, device="cuda")
    o, lse = gpu_lib.forward(_dev(q8), z8, z8, scale=0.1, q_scale=_dev(sq), k_scale=zs, v_scale=zs)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 256])
def test_fp8_zero_and_tiny_v_scales(gpu_lib, causal, d):
    """V tiles whose scale is 0, or so small against the head's largest V
    scale (w = 2^-30) that every rounded weight is 0: their keys still count
    in the softmax sum l and add nothing to O, as in the emulation."""
    q8, k8, v8, sq, sk, sv = _exact_problem(2, 2, 300, 700, seed=57, d=d)
    sv = sv.copy()
    sv[0, 0, 1] = 0.0
    sv[1, 1, 2] = sv[1, 1].max() * np.float32(2.0 ** -30)
    sv[0, 1, :] = 0.0  # a head with every V scale 0: O = 0, lse still finite
    o, lse = _run_fp8(gpu_lib, q8, k8, v8, sq, sk, sv, 0.0884, causal)
    ref = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.0884, causal, ambiguity=3e-5, parts=True, block=BLOCK[d])
    assert np.all(ref["o"][0, 1] == 0)
    _check(o, lse, ref["o"], ref["lse"], f"fp8 d{d} zero V scales causal{causal}",
           allow=ref["flip"] + _pv_bound(ref))


# Q carries values in one channel per accumulation group of the e4m3 MFMA
# (8 channels), so every group holds at most one nonzero product and
# S = K Q^T rounds only where the group sums add.


def _quantiser_problem(kind, causal, B=2, H=2, nq=1000, nk=2000, seed=0, d=128):
    """Codes and scales from the oracle's quantiser (fp32 N(0,1) inputs):
    "normal": block scales, K rotated; "outlier_block": Q and K channels 0 and
    16 scaled by 50, block scales, K rotated; "outlier_tensor": the same
    outliers, one scale per tensor, nothing rotated (the normal channels then
    take small codes and subnormals).  Q carries values only in every 8th
    channel (one per MFMA accumulation group).  Scales are arbitrary fp32
    values."""
    rng = np.random.default_rng(seed + 100 * causal + len(kind) + d)
    chans = np.arange(0, d, MFMA_GROUP)
    q = np.zeros((B, H, nq, d), np.float32)
    q[..., chans] = rng.standard_normal((B, H, nq, len(chans)), dtype=np.float32)
    k = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32)
    scale = 0.7 if kind == "normal" else 1.0 / np.sqrt(d)
    if kind != "normal":
        q[..., [0, 16]] *= 50
        k[..., [0, 16]] *= 50
    pt = kind == "outlier_tensor"
    q8, sq = F.quantize(q, None, pt)
    k8, sk = F.quantize(k, None if pt else signs, pt)
    v8, sv = F.quantize(v, None, pt)
    return q8, k8, v8, sq, sk, sv, scale


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind,d", [("normal", 128), ("outlier_block", 128), ("outlier_tensor", 128),
                                    ("normal", 64), ("outlier_block", 256)])
def test_fp8_kernel_vs_emulation_quantiser(gpu_lib, kind, d, causal):
    """Element-wise parity on codes from the quantiser (B2 H2, 1000 queries,
    2000 keys): codes up to 448, subnormal Q/K/V and P codes, non-power-of-two
    scales.  Allowance per element (``_quantiser_allowance``): the S product's
    rounding inside the MFMA (zero for these Q rows) through code flips, l and
    the integer M; the PV product's truncation (``_pv_bound``); the bf16
    rounding of O (2^-8 relative) and 2e-5 for fp32 accumulation."""
    q8, k8, v8, sq, sk, sv, scale = _quantiser_problem(kind, causal, d=d)
    assert np.any(np.abs(F.e4m3_decode(q8)) == 448) and np.any((q8 & 0x78) == 0) and np.any((v8 & 0x7F) == 0x7E)
    assert not np.all(np.log2(sk) == np.rint(np.log2(sk)))
    o, lse = _run_fp8(gpu_lib, q8, k8, v8, sq, sk, sv, scale, causal)
    ref, allow, lse_bound = _quantiser_allowance(q8, k8, v8, sq, sk, sv, scale, causal, block=BLOCK[d])
    assert np.any((ref["p8"] > 0) & (ref["p8"] < 2.0 ** -6))  # subnormal P codes occur
    tol = 2.0 ** -8 * (np.abs(ref["o"]) + allow) + allow + 2e-5
    err = np.abs(o - ref["o"])
    i = np.unravel_index(np.argmax(err / tol), err.shape)
    print(f"fp8 quantiser codes {kind} causal{causal}: max |O - O_emu| {err.max():.3e}, "
          f"worst err/tol {err[i] / tol[i]:.3f}, mean allowance {allow.mean():.2e}, mean |O| {np.abs(ref['o']).mean():.2e}")
    assert err[i] <= tol[i], f"|O - O_emu| = {err[i]:.3e} > {tol[i]:.3e} at {i}"
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(np.abs(lse - ref["lse"])[fin] <= (1e-3 * np.maximum(1.0, np.abs(ref["lse"])) + lse_bound)[fin])
    assert np.mean(allow) <= 0.1 * np.mean(np.abs(ref["o"]))  # the allowance stays a small part of the signal


# ---------------------------------------------------------------- full size, end to end

def _truth_all(q, k, v, scale, workers=4):
    """fp64 attention of the fp32 originals for every (b, h) head, one head
    per oracle call (a few heads at a time in a thread pool: the matmuls
    and exponentials release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    B, H = q.shape[:2]
    out = np.empty(q.shape, dtype=np.float64)

    def one(bh):
        b, h = divmod(bh, H)
        out[b, h] = OX.attention(q[b, h], k[b, h], v[b, h], scale)[0]

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(B * H)))
    return out


def _end_to_end(attn, w, per_tensor, inp, truth, heads=((0, 0), (1, 7), (0, 15), (1, 12)), n_rows=96):
    """Device pre-processing and attention on the fp32 inputs of workload w.
    Returns (RMSE of the whole device output against the fp64 truth, device
    RMSE and emulation RMSE on sampled rows of `heads`)."""
    q, k, v, signs = inp["q"], inp["k"], inp["v"], inp["signs"]
    sg = None if per_tensor else _dev(signs)
    q8, sq = attn.fp8_quantize(_dev(q), sg, per_tensor)
    k8, sk = attn.fp8_quantize(_dev(k), sg, per_tensor)
    v8, sv = attn.fp8_quantize(_dev(v), None, per_tensor)
    o, lse = attn.forward(q8, k8, v8, scale=w.scale, q_scale=sq, k_scale=sk, v_scale=sv)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    assert np.all(np.isfinite(o)) and torch.all(torch.isfinite(lse))
    full = F.rmse(o, truth)
    # the oracle's own pipeline (quantiser and emulation) on sampled heads and rows
    so = None if per_tensor else signs
    rq8, rsq = F.quantize(q, so, per_tensor)
    rk8, rsk = F.quantize(k, so, per_tensor)
    rv8, rsv = F.quantize(v, None, per_tensor)
    gpu_err, emu_err = [], []
    for b, h in heads:
        rows = sample_rows(w.Nq, n_rows, seed=b * 16 + h)
        emu, _ = F.attention_fp8(rq8[b, h], rk8[b, h], rv8[b, h], rsq[b, h], rsk[b, h], rsv[b, h], w.scale,
                                 rows=rows)
        gpu_err.append(o[b, h][rows] - truth[b, h][rows])
        emu_err.append(emu - truth[b, h][rows])
    g = float(np.sqrt(np.mean(np.concatenate(gpu_err) ** 2)))
    e = float(np.sqrt(np.mean(np.concatenate(emu_err) ** 2)))
    return full, g, e


def test_fp8_full_normal_rmse(gpu_lib):
    """N(0,1) inputs of the fp8 shape (B2 H16 N8192 d128): the RMSE of the
    whole device output (all 32 heads x 8192 rows x 128) against the fp64
    attention of the fp32 originals is <= 3e-2, and on sampled rows the
    device RMSE is within 10 % of the emulation's."""
    w = W.WORKLOADS["fp8_normal"]
    inp = W.make_inputs(w)
    truth = _truth_all(inp["q"], inp["k"], inp["v"], w.scale)
    full, g, e = _end_to_end(gpu_lib, w, False, inp, truth)
    print(f"fp8 N(0,1): device RMSE {full:.3e} (whole output); sampled rows {g:.3e}, emulation {e:.3e}")
    assert full <= 3e-2
    assert g <= 1.1 * e + 1e-5


def test_fp8_full_outlier_gates(gpu_lib):
    """Outlier workload (B2 H16 N8192 d128, 4 channels x50 in Q and K): over
    the whole output, the per-tensor RMSE is >= 2x the block + Hadamard RMSE;
    on sampled rows each device RMSE is within 10 % of its emulation's."""
    w = W.WORKLOADS["fp8_outlier"]
    inp = W.make_inputs(w)
    truth = _truth_all(inp["q"], inp["k"], inp["v"], w.scale)
    blk, g_blk, e_blk = _end_to_end(gpu_lib, w, False, inp, truth)
    pt, g_pt, e_pt = _end_to_end(gpu_lib, w, True, inp, truth)
    print(f"fp8 outliers, whole output: block+Hadamard RMSE {blk:.3e}, per-tensor {pt:.3e}, ratio {pt / blk:.2f}; "
          f"sampled rows: block {g_blk:.3e} (emulation {e_blk:.3e}), per-tensor {g_pt:.3e} (emulation {e_pt:.3e})")
    assert pt / blk >= 2.0
    assert g_blk <= 1.1 * e_blk and g_pt <= 1.1 * e_pt


# ---------------------------------------------------------------- variable-length batches

VARLEN_LENS = [300, 1, 0, 128, 129, 513, 100]  # ragged, a one-token and an empty sequence


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_prep_varlen_no_rotation_bitwise(gpu_lib, in_dtype, d, per_tensor):
    """Tiles restart at every sequence: codes and scales equal the oracle's
    per-sequence quantisation bit for bit, including the entries past the
    last sequence's tiles."""
    cu = W.cu_seqlens(VARLEN_LENS)
    rng = np.random.default_rng(d + 5)
    x = rng.standard_normal((3, int(cu[-1]), d), dtype=np.float32) * np.float32(2.0)
    x[1, 300:301] = 0.0  # the one-token sequence of head 1 is all zero: scale 1
    xt = torch.from_numpy(x) if in_dtype == "f32" else W.to_dtype(x, in_dtype)
    codes, scales = gpu_lib.fp8_quantize_varlen(xt.cuda(), _dev(cu), None, per_tensor)
    torch.cuda.synchronize()
    ref_codes, ref_scales = F.quantize_varlen(xt.double().numpy().astype(np.float32), cu, None, per_tensor)
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    bad = np.argwhere(codes.cpu().numpy() != ref_codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("per_tensor", [False, True])
def test_prep_varlen_many_sequences_bitwise(gpu_lib, per_tensor):
    """More sequences than a wave's 64 lanes (the slot lookup first picks a
    block of 64), empty, one-token and tile-aligned ones: codes and every
    scale entry, owned or not, equal the oracle's bit for bit."""
    lens = [int(x) for x in np.random.default_rng(19).integers(0, 300, 150)] + [0, 1, 128, 256]
    cu = W.cu_seqlens(lens)
    x = np.random.default_rng(20).standard_normal((2, int(cu[-1]), 64), dtype=np.float32)
    codes, scales = gpu_lib.fp8_quantize_varlen(torch.from_numpy(x).cuda(), _dev(cu), None, per_tensor)
    torch.cuda.synchronize()
    ref_codes, ref_scales = F.quantize_varlen(x, cu, None, per_tensor)
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)


def _exact_varlen_problem(H, lens_q, lens_k, seed, d=128):
    cq, ck = W.cu_seqlens(lens_q), W.cu_seqlens(lens_k)
    nq, nk, B = int(cq[-1]), int(ck[-1]), len(lens_q)
    q8 = W.random_codes_from(EXACT_CODES, (H, nq, d), seed)
    k8 = W.random_codes_from(EXACT_CODES, (H, nk, d), seed + 1)
    v8 = W.random_codes_from(EXACT_CODES, (H, nk, d), seed + 2)
    sq = W.random_pow2_scales((H, F.varlen_scale_len(nq, B)), seed + 3, -1, 0)
    sk = W.random_pow2_scales((H, F.varlen_scale_len(nk, B)), seed + 4, -1, 0)
    sv = W.random_pow2_scales((H, F.varlen_scale_len(nk, B)), seed + 5, -7, -4)
    return q8, k8, v8, sq, sk, sv, cq, ck


# more sequences than one wave's 64 lanes (the kernels' slot lookup then
# picks a block of 64 first), with empty and one-token ones
MANY_LENS_Q = [int(x) for x in np.random.default_rng(41).integers(0, 330, 90)] + [0, 1, 129]
MANY_LENS_K = [int(x) for x in np.random.default_rng(42).integers(0, 330, 90)] + [5, 0, 129]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens_q,lens_k,d", [(VARLEN_LENS, VARLEN_LENS, 128), ([200, 0, 300, 7], [90, 5, 400, 0], 128),
                                             (VARLEN_LENS, VARLEN_LENS, 64), (VARLEN_LENS, VARLEN_LENS, 256),
                                             (MANY_LENS_Q, MANY_LENS_K, 128)],
                         ids=["same", "q_ne_k", "same_d64", "same_d256", "many"])
def test_fp8_varlen_kernel_vs_emulation(gpu_lib, causal, lens_q, lens_k, d):
    """Each sequence against the oracle's fp8 emulation of it, with its own
    scale tiles and V-scale normalisation (same bar and allowances as the
    dense kernel test)."""
    q8, k8, v8, sq, sk, sv, cq, ck = _exact_varlen_problem(3, lens_q, lens_k, seed=len(lens_q) + 17 + d, d=d)
    o, lse = gpu_lib.forward(_dev(q8), _dev(k8), _dev(v8), causal=causal, scale=0.0884, cu_seqlens_q=_dev(cq),
                             cu_seqlens_k=_dev(ck), q_scale=_dev(sq), k_scale=_dev(sk), v_scale=_dev(sv))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and o.shape == q8.shape and lse.shape == q8.shape[:2]
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    ref_o = np.zeros(q8.shape)
    ref_l = np.full(q8.shape[:2], -np.inf)
    allow = np.zeros(q8.shape)
    for qa, r in F.attention_fp8_varlen(q8, k8, v8, sq, sk, sv, cq, ck, 0.0884, causal, ambiguity=3e-5,
                                        parts=True, block=BLOCK[d]):
        n = r["o"].shape[-2]
        ref_o[:, qa:qa + n], ref_l[:, qa:qa + n] = r["o"], r["lse"]
        allow[:, qa:qa + n] = r["flip"] + _pv_bound(r)
    _check(o, lse, ref_o, ref_l, f"fp8 varlen causal{causal}", allow=allow)
    assert np.mean(allow) <= 0.25 * np.mean(np.abs(ref_o)) + 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_varlen_end_to_end_rmse(gpu_lib, causal):
    """fp32 packed inputs -> rotation and per-sequence block quantisation ->
    fp8 attention, all on the device, against the fp64 attention of the fp32
    originals: RMSE <= 3e-2 on N(0,1) inputs, and close to the emulation's."""
    lens = [700, 129, 1, 400]
    cu = W.cu_seqlens(lens)
    T, H, d = int(cu[-1]), 4, 128
    rng = np.random.default_rng(41)
    q, k, v = (rng.standard_normal((H, T, d), dtype=np.float32) for _ in range(3))
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32)
    cud, sd = _dev(cu), _dev(signs)
    q8, sq = gpu_lib.fp8_quantize_varlen(_dev(q), cud, sd)
    k8, sk = gpu_lib.fp8_quantize_varlen(_dev(k), cud, sd)
    v8, sv = gpu_lib.fp8_quantize_varlen(_dev(v), cud, None)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward(q8, k8, v8, causal=causal, scale=scale, cu_seqlens_q=cud, cu_seqlens_k=cud,
                             q_scale=sq, k_scale=sk, v_scale=sv)
    torch.cuda.synchronize()
    truth_o, _ = oracle.attention_varlen(q, k, v, cu, cu, scale, causal)
    err = F.rmse(o.double().cpu().numpy(), truth_o)
    emu_o, _ = F.attention_fp8_varlen(q8.cpu().numpy(), k8.cpu().numpy(), v8.cpu().numpy(), sq.cpu().numpy(),
                                      sk.cpu().numpy(), sv.cpu().numpy(), cu, cu, scale, causal)
    emu = F.rmse(emu_o, truth_o)
    assert err <= 3e-2, err
    assert err <= 1.1 * emu + 1e-3, (err, emu)


def test_fp8_causal_pairs_odd_heads(gpu_lib):
    """Causal fp8 launches run two query tiles per workgroup: across heads h
    and h + heads/2 for an even head count (the tests above), within one
    head (t, T-1-t) for an odd one, with the middle tile alone when the
    tile count is odd (9 tiles of 128 rows here)."""
    q8, k8, v8, sq, sk, sv = _exact_problem(1, 3, 1100, 1100, seed=91)
    o, lse = _run_fp8(gpu_lib, q8, k8, v8, sq, sk, sv, 0.0884, True)
    ref = F.attention_fp8(q8, k8, v8, sq, sk, sv, 0.0884, True, ambiguity=3e-5, parts=True)
    allow = ref["flip"] + _pv_bound(ref)
    _check(o, lse, ref["o"], ref["lse"], "fp8 causal, 3 heads", allow=allow)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_offsets_beyond_2_31(gpu_lib, causal):
    """e4m3 Q of more than 2^31 codes (B1 H3, Nq = 2^23 + 37, d = 128: head
    2 starts at byte 2^31 + 9472) and bf16 O of more than 2^32 bytes, against
    64 keys.  Q row g (g = head * Nq + i) is row (g * 2654435761 + 12345)
    mod 4096 of a seeded bank of exact codes, gathered on the device; the Q
    tile scales are drawn per tile.  The oracle sees each sampled row as row
    0 of a 128-row tile of its own with that row's tile scale (rows >= 63
    see all 64 keys; causal rows below that are checked within tile 0)."""
    H, nq, nk, d, R = 3, 2 ** 23 + 37, 64, 128, 4096
    nt = (nq + 127) // 128
    bank = W.random_codes_from(EXACT_CODES, (R, d), 95)
    _, k8, v8, _, sk, sv = _exact_problem(1, H, 1, nk, seed=96)
    sq = W.random_pow2_scales((1, H, nt), 97, -1, 0)

    def bank_index(g):
        return (g * 2654435761 + 12345) % R

    g = torch.arange(H * nq, dtype=torch.int64, device="cuda")
    qd = _dev(bank).index_select(0, bank_index(g)).view(1, H, nq, d)
    del g
    assert qd.stride(1) * 2 > 2 ** 31
    scale = 0.0884
    o, lse = gpu_lib.forward(qd, _dev(k8), _dev(v8), causal=causal, scale=scale,
                             q_scale=_dev(sq), k_scale=_dev(sk), v_scale=_dev(sv))
    torch.cuda.synchronize()
    for h in range(H):
        rows = np.unique(np.concatenate([sample_rows(nq, 24, seed=h), np.arange(0, 64, 9), [nq - 1]]))
        ri = torch.from_numpy(rows).cuda()
        o_h = o[0, h].index_select(0, ri).double().cpu().numpy()
        l_h = lse[0, h].index_select(0, ri).double().cpu().numpy()
        far = rows >= nk - 1
        rf = rows[far]
        q_pad = np.zeros((len(rf) * 128, d), dtype=np.uint8)
        q_pad[::128] = bank[bank_index(np.int64(h) * nq + rf.astype(np.int64))]
        ref = F.attention_fp8(q_pad, k8[0, h], v8[0, h], sq[0, h][rf // 128], sk[0, h], sv[0, h], scale, False,
                              rows=np.arange(len(rf)) * 128, ambiguity=3e-5, parts=True)
        _check(o_h[far], l_h[far], ref["o"], ref["lse"], f"fp8 offsets, head {h}, causal {causal}",
               allow=ref["flip"] + _pv_bound(ref))
        near = rows[~far]
        if near.size:
            q_t0 = bank[bank_index(np.int64(h) * nq + np.arange(128, dtype=np.int64))]
            ref = F.attention_fp8(q_t0, k8[0, h], v8[0, h], sq[0, h][:1], sk[0, h], sv[0, h], scale, causal,
                                  rows=near, ambiguity=3e-5, parts=True)
            _check(o_h[~far], l_h[~far], ref["o"], ref["lse"], f"fp8 offsets tile 0, head {h}, causal {causal}",
                   allow=ref["flip"] + _pv_bound(ref))
    del qd, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 256])
def test_fp8_other_head_dims_end_to_end(gpu_lib, d, causal):
    """d = 64 and 256, all on the device (rotation, block quantisation, e4m3
    attention) from N(0,1) fp32 inputs (B1 H4 N2000): RMSE against the fp64
    attention of the originals <= 3e-2, and within 10 % (plus 1e-4) of the
    oracle's quantiser and emulation on the same inputs."""
    B, H, n = 1, 4, 2000
    rng = np.random.default_rng(d + causal)
    q, k, v = (rng.standard_normal((B, H, n, d), dtype=np.float32) for _ in range(3))
    signs = rng.choice([-1.0, 1.0], d).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    sd = _dev(signs)
    q8, sq = gpu_lib.fp8_quantize(_dev(q), sd)
    k8, sk = gpu_lib.fp8_quantize(_dev(k), sd)
    v8, sv = gpu_lib.fp8_quantize(_dev(v), None)
    o, lse = gpu_lib.forward(q8, k8, v8, causal=causal, scale=scale, q_scale=sq, k_scale=sk, v_scale=sv)
    torch.cuda.synchronize()
    truth, _ = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale, causal)
    err = F.rmse(o.double().cpu().numpy(), truth)
    (rq8, rsq), (rk8, rsk), (rv8, rsv) = F.quantize(q, signs), F.quantize(k, signs), F.quantize(v)
    emu, _ = F.attention_fp8(rq8, rk8, rv8, rsq, rsk, rsv, scale, causal, block=BLOCK[d])
    e = F.rmse(emu, truth)
    print(f"fp8 d{d} causal{causal}: device RMSE {err:.3e}, emulation {e:.3e}")
    assert err <= 3e-2
    assert err <= 1.1 * e + 1e-4


# ---------------------------------------------------------------- key chunks (attn_fwd_splitkv_fp8)

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,nq,nk,S", [(128, 300, 1000, 3), (128, 1, 2000, 8), (64, 129, 700, 4),
                                       (256, 200, 900, 5), (128, 100, 100, 4), (128, 513, 1500, 16)])
def test_fp8_splitkv_vs_emulation(gpu_lib, causal, d, nq, nk, S):
    """Every chunk's workspace rows against the oracle's emulation of that
    chunk (``attention_fp8_splitkv``: whole 128-key scale tiles, the chunk's
    own largest V scale, absolute causal indices; same allowances as the
    dense test), empty and invisible chunks as O = 0, lse = -inf; then the
    merged bf16 output against the merged emulation, allowing each chunk's
    allowance at its merge weight."""
    q8, k8, v8, sq, sk, sv = _exact_problem(2, 2, nq, nk, seed=nq + 5 * nk + d + S, d=d)
    op = torch.full((S, 2, 2, nq, d), float("nan"), device="cuda")
    lp = torch.full((S, 2, 2, nq), float("nan"), device="cuda")
    o, lse = gpu_lib.forward_splitkv_fp8(_dev(q8), _dev(sq), _dev(k8), _dev(sk), _dev(v8), _dev(sv), causal=causal,
                                         scale=0.0884, num_splits=S, o_part=op, lse_part=lp)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ref_o, ref_l, chunks = F.attention_fp8_splitkv(q8, k8, v8, sq, sk, sv, 0.0884, causal, num_splits=S,
                                                   ambiguity=3e-5, parts=True, block=BLOCK[d])
    op, lp = op.double().cpu().numpy(), lp.double().cpu().numpy()
    allow_m = np.zeros(ref_o.shape)
    for s, (kb, ke, r) in enumerate(chunks):
        what = f"fp8 split d{d} causal{causal} {nq}x{nk} S{S} chunk {s} [{kb}, {ke})"
        if r is None:
            assert np.all(np.isneginf(lp[s])) and np.all(op[s] == 0.0), what
            continue
        allow = r["flip"] + _pv_bound(r)
        _check(op[s], lp[s], r["o"], r["lse"], what, allow=allow)
        with np.errstate(invalid="ignore"):
            wgt = np.where(np.isfinite(r["lse"]), np.exp(r["lse"] - np.where(np.isfinite(ref_l), ref_l, 0.0)), 0.0)
        allow_m += wgt[..., None] * allow
    _check(o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l,
           f"fp8 split d{d} causal{causal} {nq}x{nk} S{S} merged", allow=allow_m)


def test_fp8_splitkv_end_to_end(gpu_lib):
    """Quantiser codes of N(0,1) inputs (rotation on Q and K), 8192 keys in 8
    chunks: RMSE against the fp64 attention of the originals within 10 % of
    the one-pass fp8 kernel's on the same codes, and the two outputs close."""
    B, H, nq, nk, d = 1, 4, 256, 8192, 128
    rng = np.random.default_rng(77)
    q, k, v = (rng.standard_normal((B, H, n, d), dtype=np.float32) for n in (nq, nk, nk))
    signs = _dev(rng.choice([-1.0, 1.0], d).astype(np.float32))
    scale = 1.0 / np.sqrt(d)
    q8, sq = gpu_lib.fp8_quantize(_dev(q), signs)
    k8, sk = gpu_lib.fp8_quantize(_dev(k), signs)
    v8, sv = gpu_lib.fp8_quantize(_dev(v), None)
    o1, l1 = gpu_lib.forward(q8, k8, v8, scale=scale, q_scale=sq, k_scale=sk, v_scale=sv)
    o2, l2 = gpu_lib.forward_splitkv_fp8(q8, sq, k8, sk, v8, sv, scale=scale, num_splits=8)
    torch.cuda.synchronize()
    truth, tl = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale, False)
    e1 = F.rmse(o1.double().cpu().numpy(), truth)
    e2 = F.rmse(o2.double().cpu().numpy(), truth)
    print(f"fp8 split end to end: RMSE one pass {e1:.3e}, 8 chunks {e2:.3e}")
    assert e2 <= 1.1 * e1 + 1e-4
    assert np.abs(l2.double().cpu().numpy() - tl).max() <= 2e-2
