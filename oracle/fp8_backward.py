"""The fp8 backward pass, E5M2 for the gradient operands, in float64 (test
infrastructure).

"Flash Attention 3：让 GPU 跑满的注意力计算", §4.1.2 gives the forward pass
E4M3 (4 exponent bits, 3 mantissa bits) and back-propagation E5M2 (5
exponent bits, 2 mantissa bits: more range for gradients, less precision);
the same post keeps the softmax statistics in higher precision.  It prints
no algorithm for the backward pass.  What is computed is fixed by
``oracle.backward`` (the chain rule of the forward definition):

    dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  delta_i = dO_i . O_i,
    dQ = scale dS K,  dK = scale dS^T Q,

here with the five products taken on fp8 operands.  Readings where the pages
are silent (each is listed with its reason in the design notes):

* E5M2 is the OCP format: exponent bias 15, largest finite 57344, smallest
  normal 2^-14, subnormal step 2^-16; rounding to nearest, ties to even;
  magnitudes beyond 57344 saturate to 57344 (the device clamps before it
  converts).
* Q, K, V are the e4m3 codes and per-128-row-tile scales that the fp8
  forward takes (``oracle.fp8.quantize``); the gradients are those of the
  dequantised values q = s_q decode(codes) etc.  For rotated inputs
  (Q' = QM, K' = KM) they are the gradients with respect to Q' and K';
  the gradient with respect to Q is dQ' M^T (M orthogonal).
* dO (given in 16-bit floats) is block-quantised to e5m2 like the forward
  quantises Q: one fp32 scale per (batch, head, 128-row tile),
  s = amax / 57344 (1 for an all-zero tile), code = e5m2(fp32(dO / s)).
* P = exp(S - lse) from the recomputed scores S = scale q k^T of the
  dequantised codes and the lse that the forward stored; dP = dO_q v^T
  with dO_q the dequantised e5m2 dO; delta_i = dO_i . O_i from the
  forward's O and the unquantised dO.  dS = P (dP - delta).
* The operands that the backward forms itself are rounded, and the
  per-tile scale of the operand that each product sums over is folded into
  the rounded factor (as the forward folds the V tile's scale into P), so a
  product needs no per-tile correction:
      dV = scale_do_max 2^-8 sum_q P8_qk do8_q,   P8  = e4m3(2^8 P s_do(q) / max s_do)
      dK = scale s_q_max sum_q dSq_qk q8_q,        dSq = e5m2(dS s_q(q) / max s_q)
      dQ = scale s_k_max sum_k dSk_qk k8_k,        dSk = e5m2(dS s_k(k) / max s_k)
  (max over the head's tiles; 2^8 P <= 256 stays inside e4m3).  The
  rounding decisions are taken on fp32 values, as the device does.
"""

from __future__ import annotations

import numpy as np

from .exact import _f64, scores
from .fp8 import F32_TINY, dequantize, e4m3_decode, e4m3_round_f32

E5M2_MAX = 57344.0
E5M2_MIN_NORMAL_EXP = -14
E5M2_MANT_BITS = 2
P_SCALE = 256.0  # P enters the dV product as e4m3(2^8 P ...), as in the forward


# --------------------------------------------------------------------------
# e5m2 from the format definition
# --------------------------------------------------------------------------

def e5m2_round(x) -> np.ndarray:
    """Round to the nearest e5m2 value (ties to even), saturating at +-57344.

    Binade of |x| = 2^e (e >= -14; below that the subnormal spacing of the
    -14 binade, 2^-16, applies); the spacing in the binade is 2^(e-2).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, E5M2_MIN_NORMAL_EXP)
    # floor(log2) can be off by one next to a power of two; fix it exactly.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.maximum(e, E5M2_MIN_NORMAL_EXP)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    quantum = np.ldexp(1.0, (e - E5M2_MANT_BITS).astype(np.int64))
    r = np.rint(ax / quantum) * quantum  # ties to even; ax/quantum is exact
    r = np.minimum(r, E5M2_MAX)
    r = np.where(ax == 0, 0.0, r)
    out = np.copysign(r, x)
    return np.where(np.isnan(x), np.nan, out)


def e5m2_round_f32(x32) -> np.ndarray:
    """e5m2 rounding of float32 values (the decision in fp32, as on device)."""
    return e5m2_round(np.asarray(x32, dtype=np.float32).astype(np.float64))


def e5m2_decode(codes) -> np.ndarray:
    """Value of e5m2 bit patterns (uint8) as float64 (s eeeee mm; exponent 31
    is inf for mantissa 0, else NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    ef = (c >> 2) & 0x1F
    mf = c & 0x3
    val = np.where(ef == 0, mf * 2.0 ** -16, (1.0 + mf / 4.0) * np.ldexp(1.0, ef - 15))
    val = np.where(ef == 0x1F, np.where(mf == 0, np.inf, np.nan), val)
    return sign * val


def e5m2_encode(x) -> np.ndarray:
    """Bit pattern (uint8) of values that are exactly representable in e5m2."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.int64)
    ax = np.abs(x)
    sub = ax < 2.0 ** E5M2_MIN_NORMAL_EXP
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, ax))).astype(np.int64)
    mant = np.rint((np.where(sub, 1.0, ax) / np.ldexp(1.0, e) - 1.0) * 4).astype(np.int64)
    code = np.where(sub, np.rint(ax * 2.0 ** 16).astype(np.int64), ((e + 15) << 2) | mant)
    code = (code | (sign << 7)).astype(np.uint8)
    if not np.array_equal(e5m2_decode(code), x):
        raise ValueError("e5m2_encode: value not representable")
    return code


# --------------------------------------------------------------------------
# Block quantisation of dO
# --------------------------------------------------------------------------

def quantize_e5m2(x, tile: int = 128):
    """Quantise x [..., N, d] to e5m2 with one scale per 128-row tile.

    Returns ``(codes uint8 [..., N, d], scales float32 [..., ceil(N/tile)])``,
    x ~= scales[..., n // tile] * e5m2_decode(codes[..., n, :]); s = fp32(amax
    / 57344) over the tile's fp32 values (2^-149 at least, 1 for an all-zero
    tile), code = e5m2(fp32(x / s)).
    """
    x32 = _f64(x).astype(np.float32)
    n = x32.shape[-2]
    nt = (n + tile - 1) // tile
    lead = x32.shape[:-2]
    scales = np.ones(lead + (nt,), dtype=np.float32)
    for t in range(nt):
        blk = np.abs(x32[..., t * tile:(t + 1) * tile, :])
        amax = blk.reshape(lead + (-1,)).max(axis=-1) if blk.size else np.zeros(lead, np.float32)
        s = np.where(amax > 0, np.maximum((amax / np.float32(E5M2_MAX)).astype(np.float32), F32_TINY),
                     np.float32(1.0))
        scales[..., t] = s.astype(np.float32)
    row_scale = np.repeat(scales, tile, axis=-1)[..., :n]
    y32 = (x32 / row_scale[..., None]).astype(np.float32)
    return e5m2_encode(e5m2_round_f32(y32)), scales


def dequantize_e5m2(codes, scales, tile: int = 128) -> np.ndarray:
    """scales[..., n // tile] * e5m2_decode(codes[..., n, :]) in float64."""
    vals = e5m2_decode(codes)
    n = vals.shape[-2]
    row_scale = np.repeat(np.asarray(scales, np.float64), tile, axis=-1)[..., :n]
    return vals * row_scale[..., None]


# --------------------------------------------------------------------------
# The backward pass on fp8 operands
# --------------------------------------------------------------------------

def _row_scales(scales, n: int, tile: int) -> np.ndarray:
    return np.repeat(np.asarray(scales, np.float64), tile, axis=-1)[..., :n]


def backward_fp8(q8, sq, k8, sk, v8, sv, o, lse, dout, scale: float, causal: bool = False,
                 tile: int = 128, rounding: bool = True, parts: bool = False):
    """(dQ, dK, dV) in float64 of the fp8 backward stated in the module docstring.

    q8, k8, v8: e4m3 codes [..., N, d] with scales [..., ceil(N/128)]; o (the
    forward's output), dout: [..., Nq, d]; lse [..., Nq] (natural log, -inf
    for a row with no visible key); scale the softmax scale.
    ``rounding=False`` keeps P and dS exact (the fold factors then cancel:
    the exact backward of the dequantised operands with dO quantised).
    ``parts=True`` returns a dict with the intermediate values as well:
    "do8", "sdo" (dO's codes and scales), "P", "dP", "delta", "dS", the
    pre-rounding operands "xp" (2^8 P s_do/max s_do), "xsq", "xsk", their
    rounded values "p8", "dsq", "dsk", and "fold" (the three max scales).
    """
    q, k, v = dequantize(q8, sq, tile), dequantize(k8, sk, tile), dequantize(v8, sv, tile)
    do8, sdo = quantize_e5m2(dout, tile)
    dod = dequantize_e5m2(do8, sdo, tile)
    nq, nk = q.shape[-2], k.shape[-2]
    lse = _f64(lse)
    s = scores(q, k, scale, causal)
    live = np.isfinite(lse)[..., None]
    with np.errstate(invalid="ignore"):
        p = np.where(live, np.exp(s - np.where(live, lse[..., None], 0.0)), 0.0)
    dp = np.matmul(dod, np.swapaxes(v, -1, -2))
    delta = (_f64(o) * _f64(dout)).sum(axis=-1)
    ds = p * (dp - delta[..., None])

    sdo_max = np.max(np.asarray(sdo, np.float64), axis=-1, keepdims=True)
    sq_max = np.max(np.asarray(sq, np.float64), axis=-1, keepdims=True)
    sk_max = np.max(np.asarray(sk, np.float64), axis=-1, keepdims=True)
    rdo = _row_scales(sdo, nq, tile) / sdo_max  # [..., Nq]
    rq = _row_scales(sq, nq, tile) / sq_max
    rk = _row_scales(sk, nk, tile) / sk_max  # [..., Nk]
    xp = (P_SCALE * p * rdo[..., :, None]).astype(np.float32)
    xsq = (ds * rq[..., :, None]).astype(np.float32)
    xsk = (ds * rk[..., None, :]).astype(np.float32)
    if rounding:
        p8, dsq, dsk = e4m3_round_f32(xp), e5m2_round_f32(xsq), e5m2_round_f32(xsk)
    else:
        p8 = P_SCALE * p * rdo[..., :, None]
        dsq, dsk = ds * rq[..., :, None], ds * rk[..., None, :]
    do_codes = e5m2_decode(do8)
    q_codes, k_codes = e4m3_decode(q8), e4m3_decode(k8)
    dv = sdo_max[..., None] / P_SCALE * np.matmul(np.swapaxes(p8, -1, -2), do_codes)
    dk = float(scale) * sq_max[..., None] * np.matmul(np.swapaxes(dsq, -1, -2), q_codes)
    dq = float(scale) * sk_max[..., None] * np.matmul(dsk, k_codes)
    if not parts:
        return dq, dk, dv
    return {"dq": dq, "dk": dk, "dv": dv, "do8": do8, "sdo": sdo, "P": p, "dP": dp, "delta": delta, "dS": ds,
            "xp": xp, "xsq": xsq, "xsk": xsk, "p8": p8, "dsq": dsq, "dsk": dsk,
            "fold": {"sdo_max": sdo_max, "sq_max": sq_max, "sk_max": sk_max}}
