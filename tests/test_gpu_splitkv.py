"""GPU parity of attention over key chunks (attn_fwd_splitkv) and of the
(O, lse) merge (attn_merge), against the CPU oracle.

* The merged result is compared with the oracle's full attention
  (``oracle.attention``) at the dense tolerances; the per-chunk workspace
  with the oracle's chunk partials (``oracle.splitkv``), which follow the
  same chunk bounds ceil(Nk / S).  Shapes cover decoding (one query per
  head, and a few: up to two run the decoding-shaped kernel; causal rows
  that see only the first keys), prefill with causal masks that make whole chunks invisible to some
  rows, more chunks than keys (empty chunks), and d = 64 / 128 / 256.
* The merge alone is fed random fp32 partials with -inf parts and all -inf
  rows and compared with ``oracle.splitkv.merge``.
* The decoding workload of the bench (B2 H32 Nq=1 Nk=32768 d=128) is checked
  in full: every (b, h) row against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import splitkv as SK
import workloads as W
from gpu_util import O_TOL, check, to_device

pytestmark = pytest.mark.gpu


def _run(attn, B, H, nq, nk, d, dtype, causal, splits, seed):
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal((B, H, nq, d), dtype=np.float32)
    k32 = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    v32 = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    qd, q64 = to_device(q32, dtype)
    kd, k64 = to_device(k32, dtype)
    vd, v64 = to_device(v32, dtype)
    scale = 1.0 / np.sqrt(d)
    o_part = torch.empty((splits, B, H, nq, d), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((splits, B, H, nq), dtype=torch.float32, device="cuda")
    o, lse = attn.forward_splitkv(qd, kd, vd, causal=causal, scale=scale, num_splits=splits,
                                  o_part=o_part, lse_part=lse_part)
    torch.cuda.synchronize()
    return (o.double().cpu().numpy(), lse.double().cpu().numpy(), o_part.double().cpu().numpy(),
            lse_part.double().cpu().numpy(), (q64, k64, v64, scale))


CASES = [
    # B, H, Nq, Nk, d, dtype, causal, splits
    (2, 3, 1, 1000, 128, "bf16", False, 7),
    (1, 4, 1, 4096, 128, "bf16", False, 16),
    (2, 2, 1, 300, 64, "f16", False, 3),
    (1, 2, 300, 2000, 128, "bf16", True, 5),
    (1, 2, 257, 700, 256, "bf16", False, 4),
    (2, 2, 100, 100, 128, "f16", True, 8),
    (1, 2, 10, 3, 128, "bf16", False, 6),
    (1, 1, 513, 1500, 64, "bf16", True, 3),
    (1, 2, 64, 4096, 256, "f16", True, 9),
    # at most 8 query rows per head: the decoding-shaped kernel
    (1, 3, 2, 777, 256, "bf16", True, 3),
    (2, 2, 4, 1500, 64, "bf16", True, 5),
    (1, 2, 8, 2049, 128, "f16", False, 4),
    (1, 2, 5, 600, 128, "bf16", True, 2),
    (2, 3, 8, 9, 256, "f16", True, 4),
    (1, 1, 3, 5000, 64, "f16", False, 64),
    (1, 2, 1, 500, 128, "bf16", True, 4),
    (1, 1, 2, 5, 64, "f16", False, 16),
]


@pytest.mark.parametrize("B,H,nq,nk,d,dtype,causal,splits", CASES)
def test_splitkv_vs_oracle(gpu_lib, B, H, nq, nk, d, dtype, causal, splits):
    o, lse, op, lp, (q, k, v, scale) = _run(gpu_lib, B, H, nq, nk, d, dtype, causal, splits, seed=nq + nk + d)
    ref_o, ref_l = oracle.attention(q, k, v, scale, causal)
    check(o, lse, ref_o, ref_l, dtype, f"splitkv {B}x{H}x{nq}x{nk} d{d} causal{causal} S{splits}")
    # the workspace holds each chunk's normalised O and lse
    _, _, rop, rlp = SK.attention_splitkv(q, k, v, scale, causal, splits, parts=True)
    assert np.array_equal(np.isneginf(lp), np.isneginf(rlp)), "empty-chunk pattern differs"
    fin = np.isfinite(rlp)
    rel = np.abs(lp[fin] - rlp[fin]) / np.maximum(1.0, np.abs(rlp[fin]))
    assert rel.size == 0 or rel.max() <= 1e-3
    assert np.all(op[~fin] == 0.0)
    assert np.abs(op[fin] - rop[fin]).max(initial=0.0) <= O_TOL[dtype]


def test_splitkv_no_keys(gpu_lib):
    q = torch.randn((1, 2, 5, 128), device="cuda").to(torch.bfloat16)
    z = torch.zeros((1, 2, 0, 128), device="cuda", dtype=torch.bfloat16)
    o, lse = gpu_lib.forward_splitkv(q, z, z, num_splits=4)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_splitkv_matches_single_pass(gpu_lib):
    """One chunk is the plain kernel on the whole key range; the merge of one
    part returns it.  The dense causal launch runs 128-key tiles and the key
    chunk launch 64-key tiles, so their fp32 sums differ only in order: lse
    agrees to a few fp32 ulps, O to the bf16 rounding of nearly equal values."""
    rng = np.random.default_rng(3)
    q, k, v = (to_device(rng.standard_normal((1, 4, 200, 128), dtype=np.float32), "bf16")[0] for _ in range(3))
    o1, l1 = gpu_lib.forward(q, k, v, causal=True)
    o2, l2 = gpu_lib.forward_splitkv(q, k, v, causal=True, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(torch.isneginf(l1), torch.isneginf(l2))
    assert (l1 - l2).abs().max().item() <= 8 * 2 ** -23 * max(1.0, l1.abs().max().item())
    assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -8


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("bf16", 256)])
def test_merge_vs_oracle(gpu_lib, dtype, d):
    rng = np.random.default_rng(d)
    S, B, H, nq = 5, 2, 3, 37
    op = rng.standard_normal((S, B, H, nq, d)).astype(np.float32)
    lp = (rng.standard_normal((S, B, H, nq)) * 4).astype(np.float32)
    lp[1, 0, 1, :10] = -np.inf  # empty parts
    op[1, 0, 1, :10] = 0.0
    lp[:, 1, 2, 5] = -np.inf    # a row with no key at all
    op[:, 1, 2, 5] = 0.0
    lp[3, 1, 0, :] += 60.0      # a dominant part
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    o, lse = gpu_lib.merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(), out_dtype=tdt)
    torch.cuda.synchronize()
    ref_o, ref_l = SK.merge(op.astype(np.float64), lp.astype(np.float64))
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(lse[fin] - ref_l[fin]).max() <= 1e-5 * np.maximum(1.0, np.abs(ref_l[fin])).max()
    # one rounding to fp16/bf16 of a convex combination of the parts
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert np.all(np.abs(o - ref_o) <= ulp * np.abs(ref_o) + 1e-6)
    assert np.all(o[1, 2, 5] == 0.0)


def test_decode_workload_full(gpu_lib):
    """The decoding shape measured by the bench, every row checked."""
    w = W.WORKLOADS["decode_bf16"]
    x = W.make_inputs(w)
    qd, q64 = to_device(x["q"], "bf16")
    kd, k64 = to_device(x["k"], "bf16")
    vd, v64 = to_device(x["v"], "bf16")
    o, lse = gpu_lib.forward_splitkv(qd, kd, vd, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    ref_o = np.zeros_like(o)
    ref_l = np.zeros_like(lse)
    for b in range(w.B):
        for h in range(w.H):
            ro, rl = oracle.attention(q64[b, h], k64[b, h], v64[b, h], w.scale, False)
            ref_o[b, h], ref_l[b, h] = ro, rl
    check(o, lse, ref_o, ref_l, "bf16", "decode B2 H32 Nk32768")
