"""FP8 (e4m3) pieces of the method, in float64 (test infrastructure).

Follows "FlashAttention-3" (lukebest.github.io), "Three techniques" §3 (FP8
throughput and precision):

* block quantisation: every tile gets its own scale, aligned with the
  kernel's tiling;
* incoherent processing: before quantisation, Q' = QM and K' = KM, where M
  is an orthogonal Hadamard matrix times random +-1, so (QM)(KM)^T = QK^T;
* compared with one scale per tensor, this lowers the error where some
  feature channels are outliers.

and "Flash Attention 3：让 GPU 跑满的注意力计算", §4.1.2: the forward pass uses
E4M3 (4 exponent bits, 3 mantissa bits); the softmax statistics (max and
sum) are kept in higher precision while the two products run in FP8.

Readings where the pages are silent (each is listed with its reason in the
design notes):

* E4M3 is the OCP "fn" variant: exponent bias 7, no infinities, largest
  finite 448, smallest normal 2^-6, subnormal step 2^-9; rounding is to
  nearest, ties to even; magnitudes beyond 448 saturate to 448;
* M = diag(s) H_d / sqrt(d) with H_d the Sylvester Hadamard matrix (d a
  power of two) and s the random signs; the same M for Q and K and every
  head, applied along the head dimension; V is not rotated;
* one fp32 scale per (tensor, batch, head, 128-row tile): s = amax / 448
  over the tile after rotation (amax = 0 gives s = 1), code = e4m3(x / s),
  x ~= s * code.  Per-tensor mode uses one amax over the whole tensor.  A
  tile whose amax / 448 underflows fp32 (amax < 448 * 2^-149) takes the
  smallest positive fp32, 2^-149, so that its codes stay finite (x / s is
  then exact and below 448);
* the quantisation decisions are taken in fp32, as the device does: the
  rotated values are rounded to fp32, s = fp32(amax / 448) and the code is
  the e4m3 rounding of fp32(x / s);
* in the PV product, P is rounded to e4m3 tile by tile, in the order of the
  online-softmax recurrence ("Flash Attention 3：让 GPU 跑满的注意力计算",
  §2.2: the term of key block j enters as exp(S_j - m_new) V_j, m_new the
  running max after block j).  The key blocks are the key tiles of the
  kernel's recurrence: the 128-key scale tiles for d <= 128, and 64-key
  halves of them for d = 256 (``block``); t = S log2(e) are the scores in
  base 2; M_j = max(M_{j-1}, ceil(max of t over block j)) is the running
  integer max (M = M_last = ceil(max_j t));
  w = s_v(tile) / max_tiles s_v is the tile's V scale relative to the
  largest V scale of that head.  Tile j's codes are
  P8 = e4m3(2^8 * 2^(t - M_j) * w), and they enter O with the exact factor
  2^(M_j - M); l sums the unrounded 2^(t - M);
  O = (max s_v) 2^-8 sum_j 2^(M_j - M) sum_{k in j} P8_k v8_k / l.  For codes
  in the normal range the factor is exact either way, so only weights
  below 2^-6 (in code units) depend on the tile in which M last rose.  A
  head whose V scales are all 0 has w = 0 (O = 0).  The P scale 2^8 puts
  the largest weight of a row in the tile of the largest V scale at code
  2^8 = 256 exactly when the row max is an integer, and weights down to
  2^-17 of the running max (the smallest subnormal code 2^-9, divided by
  2^8) survive the rounding.
"""

from __future__ import annotations

import numpy as np

from .exact import _f64

E4M3_MAX = 448.0
F32_TINY = np.float32(2.0 ** -149)  # smallest positive fp32 (a subnormal)
E4M3_MIN_NORMAL_EXP = -6  # smallest normal 2^-6
E4M3_MANT_BITS = 3
LOG2E = 1.4426950408889634  # log2(e)


# --------------------------------------------------------------------------
# e4m3 from the format definition
# --------------------------------------------------------------------------

def e4m3_round(x) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to even), saturating at +-448.

    Binade of |x| = 2^e (e >= -6; below that the subnormal spacing of the
    -6 binade applies); the spacing in the binade is 2^(e-3).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP)
    # floor(log2) can be off by one next to a power of two; fix it exactly.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    quantum = np.ldexp(1.0, (e - E4M3_MANT_BITS).astype(np.int64))
    r = np.rint(ax / quantum) * quantum  # np.rint: ties to even; ax/quantum is exact
    r = np.minimum(r, E4M3_MAX)
    r = np.where(ax == 0, 0.0, r)
    out = np.copysign(r, x)
    return np.where(np.isnan(x), np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """Bit pattern (uint8) of values that are exactly representable in e4m3fn."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8)
    ax = np.abs(x)
    code = np.zeros(x.shape, dtype=np.uint8)
    sub = ax < 2.0 ** E4M3_MIN_NORMAL_EXP
    # subnormal: value = mant * 2^-9
    code = np.where(sub, np.rint(ax * 2.0 ** 9).astype(np.int64), 0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, ax))).astype(np.int64)
    mant = np.rint((np.where(sub, 1.0, ax) / np.ldexp(1.0, e) - 1.0) * 8).astype(np.int64)
    norm = ((e + 7) << 3) | mant
    code = np.where(sub, code, norm).astype(np.uint8)
    back = e4m3_decode(code | (sign << 7))
    if not np.array_equal(back[~np.isnan(x)], x[~np.isnan(x)]):
        raise ValueError("e4m3_encode: value not representable")
    return (code | (sign << 7)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Value of e4m3fn bit patterns (uint8) as float64; 0x7f/0xff are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    val = np.where(ef == 0,
                   mf * 2.0 ** -9,
                   (1.0 + mf / 8.0) * np.ldexp(1.0, (ef - 7)))
    val = np.where((ef == 0xF) & (mf == 0x7), np.nan, val)
    return sign * val


def e4m3_round_f32(x32) -> np.ndarray:
    """e4m3 rounding of float32 values (the decision in fp32, as on device)."""
    return e4m3_round(np.asarray(x32, dtype=np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# Hadamard rotation
# --------------------------------------------------------------------------

def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (int64): H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis.

    log2(d) butterfly stages (a, b) -> (a + b, a - b) with stride 1, 2, 4, ...;
    the result equals x @ H_d (H_d symmetric).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def rotation_matrix(signs) -> np.ndarray:
    """M = diag(s) H_d / sqrt(d) (float64), orthogonal for s in {-1, +1}^d."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return (s[:, None] * sylvester(d)) / np.sqrt(d)


def rotate(x, signs) -> np.ndarray:
    """x' = x M along the last axis (float64)."""
    return _f64(x) @ rotation_matrix(signs)


# --------------------------------------------------------------------------
# Quantisation: block (per 128-row tile) and per tensor
# --------------------------------------------------------------------------

def quantize(x, signs=None, per_tensor: bool = False, tile: int = 128):
    """Rotate (if signs is given) and quantise x [..., N, d] to e4m3.

    Returns ``(codes uint8 [..., N, d], scales float32 [..., ceil(N/tile)])``
    with x' ~= scales[..., n // tile] * decode(codes[..., n, :]).  Decisions
    are taken in fp32: the rotated values are rounded to fp32, then
    s = fp32(amax / 448) and code = e4m3(fp32(x' / s)).
    """
    xr = rotate(x, signs) if signs is not None else _f64(x)
    x32 = xr.astype(np.float32)
    n = x32.shape[-2]
    nt = (n + tile - 1) // tile
    lead = x32.shape[:-2]
    scales = np.ones(lead + (nt,), dtype=np.float32)
    if per_tensor:
        amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
        s = max(np.float32(amax / np.float32(E4M3_MAX)), F32_TINY) if amax > 0 else np.float32(1.0)
        scales[...] = s
    else:
        for t in range(nt):
            blk = np.abs(x32[..., t * tile:(t + 1) * tile, :])
            amax = blk.reshape(lead + (-1,)).max(axis=-1) if blk.size else np.zeros(lead, np.float32)
            s = np.where(amax > 0, np.maximum((amax / np.float32(E4M3_MAX)).astype(np.float32), F32_TINY),
                         np.float32(1.0))
            scales[..., t] = s.astype(np.float32)
    row_scale = np.repeat(scales, tile, axis=-1)[..., :n]
    y32 = (x32 / row_scale[..., None]).astype(np.float32)
    codes = e4m3_encode(e4m3_round_f32(y32))
    return codes, scales


def dequantize(codes, scales, tile: int = 128) -> np.ndarray:
    """scales[..., n // tile] * decode(codes[..., n, :]) in float64."""
    vals = e4m3_decode(codes)
    n = vals.shape[-2]
    row_scale = np.repeat(np.asarray(scales, np.float64), tile, axis=-1)[..., :n]
    return vals * row_scale[..., None]


# --------------------------------------------------------------------------
# FP8 attention: what a tiled e4m3 kernel computes, emulated in float64
# --------------------------------------------------------------------------

P_SCALE_LOG2 = 8  # P is rounded as e4m3(2^8 * p), p <= 1, so codes stay <= 256


def attention_fp8(q8, k8, v8, sq, sk, sv, scale: float, causal: bool = False,
                  tile: int = 128, quantize_p: bool = True, rows=None, ambiguity=0.0,
                  parts: bool = False, p_mode: str = "folded", block=None, k_offset: int = 0):
    """fp8 attention of one or more heads: codes [..., N, d], scales [..., nt].

    S = scale * (sq q8)(sk k8)^T, softmax statistics in float64, and P
    rounded to e4m3 as stated in the module docstring.  With
    ``quantize_p=False`` P is kept exact (the method without P rounding).
    ``rows`` (query indices) restricts the output to those query rows.
    ``block`` is the key-block length of the running max (default ``tile``;
    a divisor of it).  ``k_offset`` is the absolute index of the first key
    (a chunk of a longer key range): the causal mask shows key j to query i
    iff k_offset + j <= i.  Returns float64 ``(O [..., Nq, d], lse [..., Nq])``.

    With ``ambiguity = delta > 0`` a third array [..., Nq, d] is returned:
    the largest change of O that re-rounding, to the other neighbouring code,
    every P element lying within relative distance delta of a rounding
    midpoint could cause.  A computation whose pre-rounding values differ
    from these by less than delta (relative) can land anywhere within it.
    delta may also be an array broadcastable to [..., Nq, Nk] (one relative
    distance per P element).

    ``p_mode`` selects the reading of the P rounding: "folded" (the module
    docstring: the V tile's scale enters P before rounding) or "rowmax" (the
    other plain reading: P8 = e4m3(2^8 * 2^(t - M)) for every key, and each
    key tile's partial product is multiplied by its own V scale in full
    precision, O = 2^-8 sum_tiles s_v(tile) sum_{j in tile} P8_j v8_j / l).

    ``parts=True`` returns a dict instead, with the intermediate values:
    "o", "lse", "flip" (if requested), "p8" (the rounded P in code units of
    the final M, [..., Nq, Nk]), "x" (P before rounding, in code units of its
    tile's running max), "shift" (M_j - M per key), "t" (the base-2 scores),
    "M" [..., Nq], "M_tile" (the running max per key tile), "l" [..., Nq],
    "sv_max" [...] and "v_codes" (values of the V codes); "M_tile" is per key
    block.
    """
    qd = dequantize(q8, sq, tile)
    qrow = np.arange(qd.shape[-2])
    if rows is not None:
        qrow = np.asarray(rows)
        qd = qd[..., qrow, :]
    kd = dequantize(k8, sk, tile)
    v_codes = e4m3_decode(v8)
    sv = np.asarray(sv, dtype=np.float64)
    nk = kd.shape[-2]
    s = float(scale) * np.matmul(qd, np.swapaxes(kd, -1, -2))
    if causal:
        s = np.where(int(k_offset) + np.arange(nk)[None, :] <= qrow[:, None], s, -np.inf)
    t = s * LOG2E
    tmax = t.max(axis=-1) if nk else np.full(t.shape[:-1], -np.inf)
    live = np.isfinite(tmax)
    M = np.where(live, np.ceil(np.where(live, tmax, 0.0)), 0.0)
    p = np.where(live[..., None], np.exp2(t - M[..., None]), 0.0)  # <= 1
    l = p.sum(axis=-1)
    # running integer max M_j of the key blocks, in key order
    blk = tile if block is None else int(block)
    if blk < 1 or tile % blk:
        raise ValueError("block must divide tile")
    nkt = (nk + blk - 1) // blk
    tpad = np.concatenate([t, np.full(t.shape[:-1] + (nkt * blk - nk,), -np.inf)], axis=-1)
    tile_max = tpad.reshape(t.shape[:-1] + (nkt, blk)).max(axis=-1) if nk else np.zeros(t.shape[:-1] + (0,))
    with np.errstate(invalid="ignore"):
        run = np.maximum.accumulate(np.ceil(tile_max), axis=-1) if nkt else tile_max
    Mj = np.repeat(run, blk, axis=-1)[..., :nk]  # -inf before a row's first visible key (those keys are masked)
    fin = np.isfinite(t)
    shift = np.where(fin, Mj - M[..., None], 0.0)  # <= 0, an integer
    with np.errstate(invalid="ignore"):  # masked keys: -inf - (-inf), discarded by the where
        p_tile = np.where(fin, np.exp2(np.where(fin, t - Mj, 0.0)), 0.0)  # P relative to the running max
    if p_mode not in ("folded", "rowmax"):
        raise ValueError("p_mode must be 'folded' or 'rowmax'")
    sv_max = sv.max(axis=-1) if sv.shape[-1] else np.ones(sv.shape[:-1])
    with np.errstate(invalid="ignore", divide="ignore"):
        w_tile = np.where(sv_max[..., None] > 0, sv / np.where(sv_max > 0, sv_max, 1.0)[..., None], 0.0)
    w = np.repeat(w_tile, tile, axis=-1)[..., :nk]
    # folded: the weight enters P before rounding; rowmax: after (full precision)
    pw = p_tile * w[..., None, :] if p_mode == "folded" else p_tile
    if quantize_p:
        p8_tile = e4m3_round_f32((pw * 2.0 ** P_SCALE_LOG2).astype(np.float32))
    else:
        p8_tile = pw * 2.0 ** P_SCALE_LOG2
    p8 = p8_tile * np.exp2(shift)  # in units of the final M (exact: a power of two)
    if p_mode == "folded":
        o_acc = np.matmul(p8, v_codes)
    else:
        o_acc = np.matmul(p8 * w[..., None, :], v_codes)
    flip = None
    if np.any(np.asarray(ambiguity) > 0):
        if p_mode != "folded":
            raise ValueError("the ambiguity bound follows the folded reading")
        x = pw * 2.0 ** P_SCALE_LOG2  # in the units of the running max of its tile
        with np.errstate(divide="ignore"):
            e = np.maximum(np.floor(np.log2(np.where(x > 0, x, 1.0))), E4M3_MIN_NORMAL_EXP)
        spacing = np.ldexp(1.0, (e - E4M3_MANT_BITS).astype(np.int64))
        frac = x / spacing - np.floor(x / spacing)  # position between neighbouring codes
        near_mid = np.abs(frac - 0.5) * spacing <= ambiguity * x
        # a value just below a power of two can also round across the binade edge
        flip = np.matmul(np.where(near_mid & (x > 0), spacing * np.exp2(shift), 0.0), np.abs(v_codes))
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(live[..., None],
                     o_acc * (sv_max[..., None, None] * 2.0 ** -P_SCALE_LOG2) / np.where(live, l, 1.0)[..., None],
                     0.0)
        lse = np.where(live, (M + np.log2(np.where(live, l, 1.0))) / LOG2E, -np.inf)
        if flip is not None:
            flip = np.where(live[..., None],
                            flip * (sv_max[..., None, None] * 2.0 ** -P_SCALE_LOG2) / np.where(live, l, 1.0)[..., None],
                            0.0)
    if parts:
        return {"o": o, "lse": lse, "flip": flip, "p8": p8, "l": l, "sv_max": sv_max, "v_codes": v_codes,
                "x": pw * 2.0 ** P_SCALE_LOG2, "shift": shift, "t": t, "M": M, "M_tile": run}
    if flip is not None:
        return o, lse, flip
    return o, lse


# --------------------------------------------------------------------------
# Key chunks (FlashDecoding) on fp8 operands
# --------------------------------------------------------------------------

def split_bounds_fp8(nk: int, num_splits: int, tile: int = 128):
    """Key ranges [begin, end) of the fp8 key chunks: ceil(nk / num_splits)
    keys rounded up to whole scale tiles, in order (the last chunks may be
    short or empty), so that no scale tile is cut between two chunks."""
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    n = -(-nk // num_splits) if nk > 0 else 0
    n = -(-n // tile) * tile
    return [(min(s * n, nk), min((s + 1) * n, nk)) for s in range(num_splits)]


def attention_fp8_splitkv(q8, k8, v8, sq, sk, sv, scale: float, causal: bool = False, num_splits: int = 1,
                          tile: int = 128, quantize_p: bool = True, ambiguity=0.0, parts: bool = False,
                          block=None):
    """fp8 attention over key chunks, merged ("FlashAttention-3" wiki page:
    FlashDecoding among the related techniques; the merge of "Flash Attention
    3：让 GPU 跑满的注意力计算", §2.2, as `oracle.splitkv.merge`).

    Each chunk (`split_bounds_fp8`) is the fp8 attention of its keys alone
    (`attention_fp8` of the chunk's codes and scale tiles): its own largest V
    scale for the P weights and a running max that starts at the chunk,
    with the causal mask on absolute key indices (k_offset).  A chunk with
    no visible key gives O_s = 0, lse_s = -inf.  Returns float64
    ``(O, lse)`` merged; ``parts=True`` returns ``(O, lse, chunks)`` with
    ``chunks`` a list of ``(begin, end, parts dict of attention_fp8 or None
    for an empty chunk)``.
    """
    from .splitkv import merge

    nq, nk = q8.shape[-2], k8.shape[-2]
    lead = q8.shape[:-2]
    o_parts, lse_parts, chunks = [], [], []
    for kb, ke in split_bounds_fp8(nk, num_splits, tile):
        if ke <= kb:
            o_parts.append(np.zeros(lead + (nq, q8.shape[-1])))
            lse_parts.append(np.full(lead + (nq,), -np.inf))
            chunks.append((kb, ke, None))
            continue
        ts = slice(kb // tile, -(-ke // tile))
        r = attention_fp8(q8, k8[..., kb:ke, :], v8[..., kb:ke, :], sq, sk[..., ts], sv[..., ts], scale, causal,
                          tile=tile, quantize_p=quantize_p, ambiguity=ambiguity, parts=True, block=block,
                          k_offset=kb)
        o_parts.append(r["o"])
        lse_parts.append(r["lse"])
        chunks.append((kb, ke, r))
    o, lse = merge(np.stack(o_parts), np.stack(lse_parts))
    if parts:
        return o, lse, chunks
    return o, lse


# --------------------------------------------------------------------------
# Variable-length batches: sequences packed along the token axis
# --------------------------------------------------------------------------

def varlen_scale_len(total: int, nseq: int, tile: int = 128) -> int:
    """Scale entries per head for a packed tensor of `total` tokens in `nseq`
    sequences: ceil(total / tile) + nseq, an upper bound on the tiles
    sum_b ceil(L_b / tile) that needs no sequence length."""
    return (int(total) + tile - 1) // tile + int(nseq)


def varlen_tile_offsets(cu, tile: int = 128) -> np.ndarray:
    """First scale entry of each sequence: floor(cu[b] / tile) + b, tile t of
    sequence b at that entry + t (scale tiles restart at every sequence, so
    none straddles two).  The ranges of consecutive sequences do not overlap,
    as floor(a / tile) + ceil(L / tile) <= floor((a + L) / tile) + 1, and all
    end below floor(T / tile) + nseq <= `varlen_scale_len`; a reader finds
    sequence b's entries from cu[b] alone, without the lengths of the
    sequences before it."""
    cu = np.asarray(cu, dtype=np.int64)
    return cu[:-1] // tile + np.arange(len(cu) - 1, dtype=np.int64)


def quantize_varlen(x, cu, signs=None, per_tensor: bool = False, tile: int = 128):
    """Rotate and quantise a packed tensor x [H, T, d] whose sequence b holds
    tokens [cu[b], cu[b+1]).

    Block mode: each sequence is quantised on its own (`quantize` of its
    [H, L_b, d] slice), its scales stored at entries
    varlen_tile_offsets(cu)[b] + t of a [H, varlen_scale_len] array; entries
    that no tile owns are 1.  Per-tensor mode: one scale for the
    whole tensor (as `quantize` of all of x), in every entry.
    Returns ``(codes uint8 [H, T, d], scales float32 [H, varlen_scale_len])``.
    """
    x64 = _f64(x)
    cu = np.asarray(cu, dtype=np.int64)
    H, T, d = x64.shape
    nseq = len(cu) - 1
    scales = np.ones((H, varlen_scale_len(T, nseq, tile)), dtype=np.float32)
    if per_tensor:
        codes, s = quantize(x64[None], signs, per_tensor=True, tile=tile)
        scales[...] = s.reshape(-1)[0] if s.size else np.float32(1.0)
        return codes[0], scales
    codes = np.zeros((H, T, d), dtype=np.uint8)
    offs = varlen_tile_offsets(cu, tile)
    for b in range(nseq):
        a, e = int(cu[b]), int(cu[b + 1])
        if e <= a:
            continue
        c, s = quantize(x64[:, a:e], signs, per_tensor=False, tile=tile)
        codes[:, a:e] = c
        scales[:, offs[b]:offs[b] + s.shape[-1]] = s
    return codes, scales


def attention_fp8_varlen(q8, k8, v8, sq, sk, sv, cu_q, cu_k, scale: float, causal: bool = False,
                         tile: int = 128, quantize_p: bool = True, ambiguity: float = 0.0, parts: bool = False,
                         block=None):
    """fp8 attention of a variable-length batch: codes [H, T, d] packed along
    tokens, scales [H, varlen_scale_len] laid out as by `quantize_varlen`.

    Each sequence is an independent problem ("Flash Attention 3：让 GPU 跑满的
    注意力计算", §5.2): `attention_fp8` of its slices and of its own scale
    entries (so the V-scale normalisation uses the largest V scale of that
    sequence and head), causal with indices local to the sequence.
    Returns float64 ``(O [H, Tq, d], lse [H, Tq])`` (and the flip bound with
    ``ambiguity > 0``); ``parts=True`` returns a list with, per non-empty
    query sequence, ``(first query row, parts dict of attention_fp8)``.
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    H, Tq, d = q8.shape
    o = np.zeros((H, Tq, d))
    lse = np.full((H, Tq), -np.inf)
    flip = np.zeros((H, Tq, d)) if ambiguity > 0 else None
    out_parts = []
    oq, ok = varlen_tile_offsets(cu_q, tile), varlen_tile_offsets(cu_k, tile)
    for b in range(len(cu_q) - 1):
        qa, qe, ka, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qe <= qa:
            continue
        ntq, ntk = (qe - qa + tile - 1) // tile, (ke - ka + tile - 1) // tile
        r = attention_fp8(q8[:, qa:qe], k8[:, ka:ke], v8[:, ka:ke], sq[:, oq[b]:oq[b] + ntq],
                          sk[:, ok[b]:ok[b] + ntk], sv[:, ok[b]:ok[b] + ntk], scale, causal, tile=tile,
                          quantize_p=quantize_p, ambiguity=ambiguity, parts=True, block=block)
        o[:, qa:qe] = r["o"]
        lse[:, qa:qe] = r["lse"]
        if flip is not None:
            flip[:, qa:qe] = r["flip"]
        out_parts.append((qa, r))
    if parts:
        return out_parts
    if flip is not None:
        return o, lse, flip
    return o, lse


def rmse(a, b) -> float:
    """sqrt(mean((a - b)^2)) over all elements, in float64."""
    a = _f64(a)
    b = _f64(b)
    return float(np.sqrt(np.mean((a - b) ** 2)))
