"""Helpers of the GPU parity tests: run the HIP path through the binding and
compare with the oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np

import workloads as W

# Tolerances on O (max abs error, every element) and lse (relative, floor 1).
O_TOL = {"f16": 2e-3, "bf16": 8e-3}
LSE_RTOL = 1e-3


def to_device(x: np.ndarray, dtype: str):
    """float32 host array -> rounded fp16/bf16 tensor on cuda:0, and its exact fp64 values."""
    t = W.to_dtype(x, dtype)
    return t.cuda(), t.double().numpy()


def run_dense(attn, q32, k32, v32, dtype, causal, scale=None):
    qd, q64 = to_device(q32, dtype)
    kd, k64 = to_device(k32, dtype)
    vd, v64 = to_device(v32, dtype)
    d = q32.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o, lse = attn.forward(qd, kd, vd, causal=causal, scale=scale)
    import torch

    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), (q64, k64, v64, scale)


def check(o, lse, o_ref, lse_ref, dtype, what=""):
    """O within the dtype's max-abs bar; lse within 1e-3 relative (floor 1); -inf matches -inf."""
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape
    assert not np.any(np.isnan(o)), f"{what}: NaN in O"
    assert not np.any(np.isnan(lse)), f"{what}: NaN in lse"
    err = np.abs(o - o_ref)
    tol = O_TOL[dtype]
    if err.size:
        i = np.unravel_index(np.argmax(err), err.shape)
        assert err[i] <= tol, f"{what}: max |O - O_ref| = {err[i]:.3e} at {i} (ref {o_ref[i]:.4f}) > {tol}"
    neg = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf pattern of lse differs"
    fin = ~neg
    if np.any(fin):
        rel = np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        assert rel.max() <= LSE_RTOL, f"{what}: lse rel err {rel.max():.3e} > {LSE_RTOL}"
    return float(err.max()) if err.size else 0.0


def sample_rows(n: int, count: int, seed: int, tile: int = 128) -> np.ndarray:
    """Query rows to check at full size: both ends, tile edges, and random rows."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, n - 1, n - 2] + [t * tile + o for t in range(0, (n + tile - 1) // tile, max(1, n // tile // 4))
                                    for o in (0, tile - 1)]
    rows = np.unique(np.clip(np.concatenate([edges, rng.integers(0, n, count)]), 0, n - 1))
    return rows
