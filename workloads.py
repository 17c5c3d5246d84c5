"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and builds the workload shapes.  It
holds none of the attention arithmetic: no softmax, no rotation, no
quantisation.  Both the CPU oracle (``oracle/``) and the HIP path receive
their inputs from here, so neither side ever produces the other's inputs.

Draw order for one workload (one ``numpy.random.default_rng(seed)``):

1. variable-length batches: the sequence lengths, ``integers(lo, hi+1, size)``;
2. Q, K, V as ``standard_normal(shape, float32)``, in that order;
3. outlier channels (fp8 workload): ``choice(d, n_outliers, replace=False)``;
4. the random +-1 signs of the Hadamard rotation: ``choice([-1, 1], d)``.

Casting fp32 -> fp16/bf16 uses torch's round-to-nearest-even ``.to()``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem.

    Dense problems use ``[B, H, N, d]``; variable-length problems pack the
    sequences along the token axis as ``[H, T, d]`` with ``cu_seqlens``
    prefix sums ``[0, L0, L0+L1, ...]``.
    """

    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "f16" | "bf16" | "fp8"
    causal: bool
    seed: int = 0
    lengths: Optional[tuple] = None  # varlen only: per-sequence lengths (q == k)
    outliers: int = 0  # fp8 workload: channels scaled by outlier_factor in Q and K
    outlier_factor: float = 50.0
    len_range: Optional[tuple] = None  # varlen: (lo, hi) the lengths were drawn from

    @property
    def varlen(self) -> bool:
        return self.lengths is not None

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def flops(self) -> float:
        """Operations of the two contractions, 4*Nq*Nk*d per head, halved if causal."""
        if self.varlen:
            tot = sum(4.0 * self.H * L * L * self.d for L in self.lengths)
        else:
            tot = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return tot / 2.0 if self.causal else tot


def varlen_lengths(n_seq: int, lo: int, hi: int, seed: int) -> tuple:
    rng = np.random.default_rng(seed)
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n_seq))


def _varlen_workload(name, n_seq, lo, hi, H, d, dtype, causal, seed):
    lengths = varlen_lengths(n_seq, lo, hi, seed)
    T = int(sum(lengths))
    return Workload(name, n_seq, H, T, T, d, dtype, causal, seed, lengths=lengths,
                    len_range=(lo, hi))


def varlen_workload(lengths, H, d, dtype="bf16", causal=True, seed=0, name="varlen"):
    """A variable-length problem with given per-sequence lengths (q == k)."""
    lengths = tuple(int(x) for x in lengths)
    T = int(sum(lengths))
    return Workload(name, len(lengths), H, T, T, d, dtype, causal, seed, lengths=lengths)


# The workloads: tiny fp16; dense bf16 (both causal modes); large head dim;
# variable length causal; fp8 with outlier features; and the bf16 shape of
# the fp8 workload (hdim 128, N 8192, non-causal).
WORKLOADS = {
    "tiny_f16": Workload("tiny_f16", 1, 2, 256, 256, 64, "f16", False),
    "dense_bf16": Workload("dense_bf16", 2, 16, 4096, 4096, 128, "bf16", False),
    "dense_bf16_causal": Workload("dense_bf16_causal", 2, 16, 4096, 4096, 128, "bf16", True),
    "hdim256_bf16": Workload("hdim256_bf16", 1, 16, 8192, 8192, 256, "bf16", False),
    "varlen_bf16_causal": _varlen_workload("varlen_bf16_causal", 8, 512, 4096, 32, 128, "bf16", True, 0),
    "fp8_outlier": Workload("fp8_outlier", 2, 16, 8192, 8192, 128, "fp8", False, outliers=4),
    "fp8_normal": Workload("fp8_normal", 2, 16, 8192, 8192, 128, "fp8", False),
    "n8k_bf16": Workload("n8k_bf16", 2, 16, 8192, 8192, 128, "bf16", False),
    # decoding: one query per (batch, head) against a long key cache
    "decode_bf16": Workload("decode_bf16", 2, 32, 1, 32768, 128, "bf16", False),
}


def cu_seqlens(lengths) -> np.ndarray:
    """``[0, L0, L0+L1, ...]`` as int32 (B+1 entries)."""
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


def qkv_fp32(w: Workload, rng: Optional[np.random.Generator] = None):
    """Q, K, V as float32 N(0,1), with the outlier channels applied.

    Returns ``(q, k, v, outlier_channels)``.  The outlier channels (same
    indices for Q and K, every head and row) are multiplied by
    ``outlier_factor``; V stays plain N(0,1).
    """
    if rng is None:
        rng = np.random.default_rng(w.seed)
        if w.len_range is not None:  # documented draw order: lengths come first
            lo, hi = w.len_range
            drawn = rng.integers(lo, hi + 1, size=len(w.lengths))
            assert tuple(int(x) for x in drawn) == tuple(w.lengths)
    if w.varlen:
        qs = (w.H, w.Nq, w.d)
        ks = (w.H, w.Nk, w.d)
    else:
        qs = (w.B, w.H, w.Nq, w.d)
        ks = (w.B, w.H, w.Nk, w.d)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    ch = np.zeros(0, dtype=np.int64)
    if w.outliers:
        ch = np.sort(rng.choice(w.d, w.outliers, replace=False))
        q[..., ch] *= np.float32(w.outlier_factor)
        k[..., ch] *= np.float32(w.outlier_factor)
    return q, k, v, ch, rng


def hadamard_signs(d: int, rng: np.random.Generator) -> np.ndarray:
    """Random +-1 signs (float32) for the rotation ``diag(s) H_d / sqrt(d)``."""
    return rng.choice(np.array([-1.0, 1.0], dtype=np.float32), d).astype(np.float32)


def make_inputs(w: Workload) -> dict:
    """All inputs of a workload, host side.

    Keys: ``q, k, v`` (float32), ``signs`` (fp8 only), ``cu_seqlens`` (varlen
    only), ``outlier_channels``.
    """
    q, k, v, ch, rng = qkv_fp32(w)
    out = {"q": q, "k": k, "v": v, "outlier_channels": ch}
    if w.dtype == "fp8":
        out["signs"] = hadamard_signs(w.d, rng)
    if w.varlen:
        out["cu_seqlens"] = cu_seqlens(w.lengths)
    return out


def to_dtype(x: np.ndarray, dtype: str):
    """Round a float32 array to fp16/bf16 (RNE) as a CPU torch tensor."""
    import torch

    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdt)


def random_problem(B, H, Nq, Nk, d, seed, dtype="bf16"):
    """Small seeded N(0,1) problem for parity sweeps: returns float32 q, k, v."""
    w = Workload("sweep", B, H, Nq, Nk, d, dtype, False, seed)
    q, k, v, _, _ = qkv_fp32(w)
    return q, k, v


def random_e4m3_codes(shape, seed, max_exp_field=10) -> np.ndarray:
    """Random e4m3fn bit patterns (uint8) with a bounded exponent field.

    Built from independent sign, exponent and mantissa integers, so the
    values lie in [-2^(max_exp_field-7) * 1.875, +...]; exponent field 15 is
    never drawn, so there are no NaN codes.
    """
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
    expo = rng.integers(0, max_exp_field + 1, size=shape, dtype=np.uint8)
    mant = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign << 7) | (expo << 3) | mant


def random_codes_from(codes, shape, seed) -> np.ndarray:
    """Uniform random choice (uint8) among the given e4m3 bit patterns."""
    rng = np.random.default_rng(seed)
    return rng.choice(np.asarray(codes, dtype=np.uint8), size=shape)


def random_pow2_scales(shape, seed, lo_exp=-3, hi_exp=0) -> np.ndarray:
    """Scales 2^e with e drawn uniformly from [lo_exp, hi_exp] (float32)."""
    rng = np.random.default_rng(seed)
    return np.ldexp(np.float32(1.0), rng.integers(lo_exp, hi_exp + 1, size=shape)).astype(np.float32)


def random_scales(shape, seed, lo=0.01, hi=0.05) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=shape).astype(np.float32)
