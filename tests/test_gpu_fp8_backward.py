"""GPU parity of the fp8 backward (attn_bwd_fp8) against the fp64 oracle
``oracle.fp8_backward``.

* dO's e5m2 quantisation takes every decision on the same fp32 values as the
  oracle (bf16 dO is exact in fp32; amax / 57344 and dO / s are correctly
  rounded), so the do8 codes and the do_scale workspace must be
  bit-identical; delta (an fp32 sum of 128 products) within 2^-17 of
  sum |o dout|.
* Gradients, element by element against the oracle on the same inputs: Q, K,
  V codes drawn from {+-1, +-1.5, +-2, +-3, +-4} with power-of-two tile
  scales, so the MFMA adds the S = Q K^T products exactly; o and lse from the
  oracle's exact forward (o rounded to bf16, lse to fp32, the same values on
  both sides); dO either "narrow" (each tile's e5m2 codes within
  [2^12, 57344], so dP = dO V^T is exact too) or N(0,1) with per-tile
  magnitudes.  The kernel forms P and dS in fp32 and rounds them to e4m3 and
  e5m2; the oracle forms them in fp64.  An error model bounds the device's
  pre-rounding value x by x_oracle +- b (the fp32 score and exp2, the fp32
  delta, the scale products and, for N(0,1) dO, the truncation of the dP
  products in the MFMA), and any code in [round(x - b), round(x + b)] is
  valid.  The allowance of an output element is the sum over its terms of
  the largest such code change times the other operand, plus the MFMA's
  truncation of the dV, dK, dQ products themselves (every product other
  than its 8-product group's largest loses less than 2^(e - 13), e the
  exponent of the group's largest product; a group lies in one aligned
  16-row block of the summed index) and the fp32 accumulation; the bf16
  output rounding adds 2^-8 of the value.
* End to end: N(0,1) inputs quantised by the oracle, the device gradients'
  RMSE against the exact gradients of the dequantised inputs is within 10 %
  (plus 2e-3) of the oracle's own.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as BW
from oracle import fp8 as F
from oracle import fp8_backward as FB
import workloads as W

pytestmark = pytest.mark.gpu

D = 128
TILE = 128
EXACT_CODES = [0x38, 0x3C, 0x40, 0x44, 0x48, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8]  # +-1, 1.5, 2, 3, 4
KEEP_BITS = 13  # the fp8 MFMA truncates products 13 bits below its group's largest
ACC = 2.0 ** -22  # fp32 accumulation of at most a few thousand terms, relative to sum |terms|


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _nt(n):
    return (n + TILE - 1) // TILE


def _dout(kind, lead, nq, seed):
    """bf16 dO [lead..., nq, 128] as a CPU tensor."""
    rng = np.random.default_rng(seed)
    if kind == "narrow":
        # e5m2 values of magnitude 2^12 .. 57344 times 2^e per tile, each tile's
        # first element 57344 * 2^e: scales 2^e, codes the values themselves
        mant = rng.choice([1.0, 1.25, 1.5, 1.75], size=lead + (nq, D))
        expo = rng.integers(12, 16, size=lead + (nq, D))
        x = mant * np.ldexp(1.0, expo) * rng.choice([-1.0, 1.0], size=lead + (nq, D))
        x = np.minimum(x, 57344.0)
        for t in range(_nt(nq)):
            x[..., t * TILE, 0] = 57344.0
            x[..., t * TILE:(t + 1) * TILE, :] *= np.ldexp(1.0, rng.integers(-22, -14, size=lead))[..., None, None]
    else:
        x = rng.standard_normal(lead + (nq, D))
        for t in range(_nt(nq)):
            x[..., t * TILE:(t + 1) * TILE, :] *= np.exp(rng.standard_normal(lead))[..., None, None]
    t = _bf16(x)
    assert kind != "narrow" or np.array_equal(t.double().numpy(), x)
    return t


def _problem(B, H, nq, nk, seed, causal, scale, do_kind):
    lead = (B, H)
    q8 = W.random_codes_from(EXACT_CODES, lead + (nq, D), seed)
    k8 = W.random_codes_from(EXACT_CODES, lead + (nk, D), seed + 1)
    v8 = W.random_codes_from(EXACT_CODES, lead + (nk, D), seed + 2)
    sq = W.random_pow2_scales(lead + (_nt(nq),), seed + 3, -2, 0)
    sk = W.random_pow2_scales(lead + (_nt(nk),), seed + 4, -2, 0)
    sv = W.random_pow2_scales(lead + (_nt(nk),), seed + 5, -6, -3)
    qd, kd, vd = F.dequantize(q8, sq), F.dequantize(k8, sk), F.dequantize(v8, sv)
    o, lse = oracle.attention(qd, kd, vd, scale, causal)
    o16 = _bf16(o)
    lse32 = lse.astype(np.float32)
    do16 = _dout(do_kind, lead, nq, seed + 6)
    return dict(q8=q8, k8=k8, v8=v8, sq=sq, sk=sk, sv=sv, o16=o16, lse32=lse32, do16=do16, qd=qd, kd=kd, vd=vd)


def _run(attn, pr, scale, causal):
    ws = (torch.full((3,) + pr["lse32"].shape, float("nan"), dtype=torch.float32, device="cuda"),
          torch.full(pr["q8"].shape, 0xFF, dtype=torch.uint8, device="cuda"),
          torch.full(pr["lse32"].shape[:-1] + (_nt(pr["q8"].shape[-2]),), float("nan"), dtype=torch.float32,
                     device="cuda"))
    dq, dk, dv = attn.backward_fp8(_dev(pr["q8"]), _dev(pr["sq"]), _dev(pr["k8"]), _dev(pr["sk"]), _dev(pr["v8"]),
                                   _dev(pr["sv"]), pr["o16"].cuda(), _dev(pr["lse32"]), pr["do16"].cuda(),
                                   causal=causal, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert g.dtype == torch.bfloat16
    out = tuple(g.double().cpu().numpy() for g in (dq, dk, dv))
    return out, tuple(w.cpu().numpy() for w in ws)


def _oracle(pr, scale, causal):
    o64 = pr["o16"].double().numpy()
    return FB.backward_fp8(pr["q8"], pr["sq"], pr["k8"], pr["sk"], pr["v8"], pr["sv"], o64,
                           pr["lse32"].astype(np.float64), pr["do16"].double().numpy(), scale, causal, parts=True)


# ------------------------------------------------------------ allowances

def _rows(s, n):
    return np.repeat(np.asarray(s, np.float64), TILE, axis=-1)[..., :n]


def _code_range(x, b, rnd):
    """Largest code change, and largest code magnitude, over values x +- b."""
    r0, lo, hi = rnd(x), rnd(x - b), rnd(x + b)
    return np.maximum(np.abs(hi - r0), np.abs(lo - r0)), np.maximum(np.abs(lo), np.abs(hi))


def _trunc_blocks(prod, axis):
    """MFMA truncation bound of sums of prod (>= 0) along `axis`: per aligned
    16-block, (nonzero count - 1) 2^(e - 13), e the exponent of its largest."""
    prod = np.moveaxis(prod, axis, -1)
    tot = np.zeros(prod.shape[:-1])
    for j0 in range(0, prod.shape[-1], 16):
        blk = prod[..., j0:j0 + 16]
        m = blk.max(-1)
        cnt = np.count_nonzero(blk, axis=-1)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        tot += np.where(cnt > 1, (cnt - 1) * np.exp2(e - KEEP_BITS), 0.0)
    return tot


def _dp_trunc(doc, vc):
    """Bound on the raw dP = do8 v8^T error in the MFMA (groups of 8
    consecutive channels) and its fp32 accumulation: [..., Nq, Nk]."""
    tot = np.zeros(doc.shape[:-1] + (vc.shape[-2],))
    for g in range(D // 8):
        sl = slice(8 * g, 8 * g + 8)
        prod = np.abs(doc[..., :, None, sl] * vc[..., None, :, sl])
        m = prod.max(-1)
        cnt = np.count_nonzero(prod, axis=-1)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        tot += np.where(cnt > 1, (cnt - 1) * np.exp2(e - KEEP_BITS), 0.0)
    return tot + ACC * np.matmul(np.abs(doc), np.swapaxes(np.abs(vc), -1, -2))


def _allowance(pr, parts, scale):
    """Per-element allowances (dq, dk, dv) of the device against the oracle."""
    nq, nk = pr["q8"].shape[-2], pr["k8"].shape[-2]
    P, dP, delta, dS = parts["P"], parts["dP"], parts["delta"], parts["dS"]
    lse = pr["lse32"].astype(np.float64)
    fin = np.isfinite(lse)
    lse2 = np.abs(np.where(fin, lse, 0.0)) * F.LOG2E
    cs = scale * F.LOG2E * _rows(pr["sq"], nq)[..., :, None] * _rows(pr["sk"], nk)[..., None, :]
    qc, kc, vc = F.e4m3_decode(pr["q8"]), F.e4m3_decode(pr["k8"]), F.e4m3_decode(pr["v8"])
    t = np.abs(np.matmul(qc, np.swapaxes(kc, -1, -2))) * cs  # |score| in base 2
    # P: the fp32 score, S * cs and lse log2(e) (a few roundings each), the
    # exponent's fma and exp2's own error (a few ulps), generously
    eps_p = np.log(2.0) * 2.0 ** -21 * (t + 2 * lse2[..., None]) + 2.0 ** -20
    sdo, fold = parts["sdo"], parts["fold"]
    rdo = _rows(sdo, nq) / fold["sdo_max"]
    rq = _rows(pr["sq"], nq) / fold["sq_max"]
    rk = _rows(pr["sk"], nk) / fold["sk_max"]
    # dS: dP from the MFMA (truncation, fp32 scale products), delta in fp32
    doc = FB.e5m2_decode(parts["do8"])
    ddp = _dp_trunc(doc, vc) * _rows(sdo, nq)[..., :, None] * _rows(pr["sv"], nk)[..., None, :]
    sum_od = np.abs(pr["o16"].double().numpy() * pr["do16"].double().numpy()).sum(-1)
    ddelta = 2.0 ** -17 * sum_od
    b_ds = np.abs(P) * (np.abs(dP) * 2.0 ** -21 + ddp + ddelta[..., None]
                        + np.abs(dP - delta[..., None]) * (eps_p + 2.0 ** -21))
    xp = FB.P_SCALE * P * rdo[..., :, None]
    xsq, xsk = dS * rq[..., :, None], dS * rk[..., None, :]
    dp8, mp8 = _code_range(xp, np.abs(xp) * (eps_p + 2.0 ** -21), F.e4m3_round)
    dsq, msq = _code_range(xsq, b_ds * rq[..., :, None] + np.abs(xsq) * 2.0 ** -22, FB.e5m2_round)
    dsk, msk = _code_range(xsk, b_ds * rk[..., None, :] + np.abs(xsk) * 2.0 ** -22, FB.e5m2_round)
    T = lambda a: np.swapaxes(a, -1, -2)  # noqa: E731
    amax = lambda c: np.abs(c).max(-1)  # noqa: E731

    def side(dcode, mcode, other, other_max, axis_sum, factor):
        # flips + MFMA truncation + accumulation, in output units
        if axis_sum == -2:  # sum over queries: [.., Nk, d]
            flips = np.matmul(T(dcode), np.abs(other))
            trunc = _trunc_blocks(mcode * other_max[..., :, None], -2)[..., :, None]
            acc = ACC * np.matmul(T(mcode), np.abs(other))
        else:  # sum over keys: [.., Nq, d]
            flips = np.matmul(dcode, np.abs(other))
            trunc = _trunc_blocks(mcode * other_max[..., None, :], -1)[..., :, None]
            acc = ACC * np.matmul(mcode, np.abs(other))
        return factor[..., None, None] * (flips + trunc + acc)

    a_dv = side(dp8, mp8, doc, amax(doc), -2, fold["sdo_max"][..., 0] / FB.P_SCALE)
    a_dk = side(dsq, msq, qc, amax(qc), -2, scale * fold["sq_max"][..., 0])
    a_dq = side(dsk, msk, kc, amax(kc), -1, scale * fold["sk_max"][..., 0])
    return a_dq, a_dk, a_dv


def _check(got, ref, allow, what):
    for name, g, r, a in zip(("dq", "dk", "dv"), got, ref, allow):
        assert g.shape == r.shape, (what, name)
        assert not np.any(np.isnan(g)), f"{what} {name}: NaN"
        # bf16 rounding of the result (half an ulp: 2^-8 of the value at most)
        err = np.abs(g - r) - a * (1 + 2.0 ** -8) - 2.0 ** -8 * np.abs(r) - 1e-30
        if err.size:
            i = np.unravel_index(np.argmax(err), err.shape)
            assert err[i] <= 0, (f"{what} {name}: |got - ref| = {abs(g[i] - r[i]):.4e} at {i} (ref {r[i]:.4e}, "
                                 f"allowance {a[i]:.3e})")


# ------------------------------------------------------------ tests

@pytest.mark.parametrize("do_kind", ["narrow", "normal"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (64, 64), (100, 100), (128, 128), (129, 300), (300, 129), (500, 700)])
def test_bwd_fp8_vs_oracle(gpu_lib, causal, nq, nk, do_kind):
    scale = 0.0884
    pr = _problem(2, 2, nq, nk, seed=nq + 7 * nk + causal, causal=causal, scale=scale, do_kind=do_kind)
    got, ws = _run(gpu_lib, pr, scale, causal)
    parts = _oracle(pr, scale, causal)
    what = f"fp8 bwd causal={causal} {nq}x{nk} dO {do_kind}"
    # workspace: dO codes and scales bit for bit; lse log2(e) as one fp32
    # product; delta within its fp32 sum, and its folded copy
    assert np.array_equal(ws[1], parts["do8"]), f"{what}: dO codes differ"
    assert np.array_equal(ws[2], parts["sdo"]), f"{what}: dO scales differ"
    assert np.array_equal(ws[0][0], pr["lse32"] * np.float32(F.LOG2E)), f"{what}: lse log2(e)"
    sum_od = np.abs(pr["o16"].double().numpy() * pr["do16"].double().numpy()).sum(-1)
    assert np.all(np.abs(ws[0][1] - parts["delta"]) <= 2.0 ** -17 * sum_od + 1e-30), f"{what}: delta"
    fq = _rows(pr["sq"], nq) / parts["fold"]["sq_max"]
    assert np.all(np.abs(ws[0][2] - parts["delta"] * fq) <= 2.0 ** -17 * sum_od * fq + 1e-30), f"{what}: delta f_q"
    allow = _allowance(pr, parts, scale)
    _check(got, (parts["dq"], parts["dk"], parts["dv"]), allow, what)
    if nk > 1:  # one key: dQ = dK = 0 (dP = delta), nothing to compare the allowance with
        for a, r in zip(allow, (parts["dq"], parts["dk"], parts["dv"])):
            assert np.mean(a) <= 0.25 * np.mean(np.abs(r)), f"{what}: allowance too large to be a check"


def test_bwd_fp8_do_quantisation_range(gpu_lib):
    """Tiny, large and all-zero dO tiles: codes and scales still bit-identical."""
    rng = np.random.default_rng(5)
    nq, nk = 512, 256
    pr = _problem(1, 2, nq, nk, seed=9, causal=False, scale=0.1, do_kind="normal")
    x = rng.standard_normal((1, 2, nq, D))
    x[0, 0, 0:128] *= 1e-30
    x[0, 0, 128:256] *= 3e3
    x[0, 1, 256:384] = 0.0
    pr["do16"] = _bf16(x)
    _, ws = _run(gpu_lib, pr, 0.1, False)
    ref8, refs = FB.quantize_e5m2(pr["do16"].double().numpy())
    assert np.array_equal(ws[1], ref8)
    assert np.array_equal(ws[2], refs)
    assert ws[2][0, 1, 2] == 1.0


def test_bwd_fp8_empty_sides(gpu_lib):
    """Nk = 0: dQ = 0; Nq = 0: dK = dV = 0."""
    pr = _problem(1, 2, 200, 1, seed=3, causal=False, scale=0.1, do_kind="normal")
    ws = (torch.empty((3, 1, 2, 200), dtype=torch.float32, device="cuda"),
          torch.empty((1, 2, 200, D), dtype=torch.uint8, device="cuda"),
          torch.empty((1, 2, 2), dtype=torch.float32, device="cuda"))
    e8 = torch.empty((1, 2, 0, D), dtype=torch.uint8, device="cuda")
    es = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    dq = torch.full((1, 2, 200, D), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 2, 200), float("-inf"), dtype=torch.float32, device="cuda")
    gpu_lib.backward_fp8(_dev(pr["q8"]), _dev(pr["sq"]), e8, es, e8, es, pr["o16"].cuda() * 0, lse,
                         pr["do16"].cuda(), scale=0.1, dq=dq, workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq).item() == 0
    dk = torch.full((1, 2, 300, D), 7.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full((1, 2, 300, D), 7.0, dtype=torch.bfloat16, device="cuda")
    e16 = torch.empty((1, 2, 0, D), dtype=torch.bfloat16, device="cuda")
    k8 = _dev(W.random_codes_from(EXACT_CODES, (1, 2, 300, D), 4))
    ks = _dev(W.random_pow2_scales((1, 2, 3), 5))
    gpu_lib.backward_fp8(e8, es, k8, ks, k8, ks, e16, torch.empty((1, 2, 0), dtype=torch.float32, device="cuda"),
                         e16, scale=0.1, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_fp8_end_to_end_rmse(gpu_lib, causal):
    """N(0,1) inputs quantised by the oracle (arbitrary e4m3 codes, fp32
    scales), N(0,1) dO: the device's gradients are as close to the exact
    gradients of the dequantised inputs as the oracle's fp8 emulation."""
    B, H, n = 1, 2, 1024
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(21 + causal)
    q, k, v = (rng.standard_normal((B, H, n, D)) for _ in range(3))
    (q8, sq), (k8, sk), (v8, sv) = F.quantize(q), F.quantize(k), F.quantize(v)
    qd, kd, vd = F.dequantize(q8, sq), F.dequantize(k8, sk), F.dequantize(v8, sv)
    o, lse = oracle.attention(qd, kd, vd, scale, causal)
    pr = dict(q8=q8, k8=k8, v8=v8, sq=sq, sk=sk, sv=sv, o16=_bf16(o), lse32=lse.astype(np.float32),
              do16=_bf16(rng.standard_normal((B, H, n, D))))
    got, _ = _run(gpu_lib, pr, scale, causal)
    emu = _oracle(pr, scale, causal)
    exact = BW.attention_backward(qd, kd, vd, pr["do16"].double().numpy(), scale, causal)
    for name, g, e, x in zip(("dq", "dk", "dv"), got, (emu["dq"], emu["dk"], emu["dv"]), exact):
        rms = np.sqrt(np.mean(x ** 2))
        r_dev = np.sqrt(np.mean((g - x) ** 2)) / rms
        r_emu = np.sqrt(np.mean((e - x) ** 2)) / rms
        assert r_dev <= 1.1 * r_emu + 2e-3, f"{name}: device rel RMSE {r_dev:.4e}, oracle {r_emu:.4e}"
        assert r_emu < 0.1, f"{name}: emulation rel RMSE {r_emu:.3e}"
