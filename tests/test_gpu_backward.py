"""GPU parity of the attention backward (attn_bwd) against the CPU oracle.

The forward runs on the GPU (its O and lse are the backward's inputs, as in
training); the gradients are compared with ``oracle.backward`` on the exact
fp16/bf16 values of q, k, v and dO.

Tolerance, element by element, from the arithmetic of the kernels (u = unit
roundoff of the storage type: 2^-8 bf16, 2^-11 fp16):

* P is recomputed from the forward's lse: relative error eps_i = |lse_i -
  lse_ref_i| + 2^-20 (2 + |lse_i|) (the lse difference, plus rounding of the
  fp32 exponent argument and of exp2);
* P enters dV = P^T dO rounded to the storage type: relative u;
* delta is read from the forward's rounded O: |ddelta_i| <= sum_c |dO_ic|
  |O_ic - O_ref_ic| (+ fp32 summation);
* dS = P (dP - delta) enters dQ and dK rounded to the storage type
  (relative u; fp16 adds 2^-25 absolute for subnormals);
* the outputs are rounded once more (relative u).

So |err dV| <= sum_i P_ij (u + eps_i) |dO_ic| + u |dV|, and for dQ, dK the
bound on each dS error, |ddS_ij| <= P_ij (eps_i |dP_ij - delta_i| +
|ddelta_i|) + u |dS_ij| (+ 2^-25), carried through the products with |K|,
|Q| and the scale.  The test allows twice that (fp32 accumulation and
second-order terms) plus 1e-6 of the largest reference value.  Each
gradient's largest ratio err / bound is printed.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as BW
import workloads as W
from gpu_util import to_device

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _inputs(B, H, nq, nk, d, dtype, seed):
    rng = np.random.default_rng(seed)
    shp_q, shp_k = (B, H, nq, d), (B, H, nk, d)
    q = to_device(rng.standard_normal(shp_q, dtype=np.float32), dtype)
    k = to_device(rng.standard_normal(shp_k, dtype=np.float32), dtype)
    v = to_device(rng.standard_normal(shp_k, dtype=np.float32), dtype)
    do = to_device(rng.standard_normal(shp_q, dtype=np.float32), dtype)
    return q, k, v, do


def _gpu(attn, q, k, v, do, scale, causal):
    o, lse = attn.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = attn.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()  # noqa: E731
    return f(o), f(lse), f(dq), f(dk), f(dv)


def bounds(q, k, v, do, o_gpu, lse_gpu, scale, causal, dtype):
    """Element-wise error bounds of (dQ, dK, dV) (see the module docstring)."""
    u = U[dtype]
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    dq, dk, dv = BW.attention_backward(q, k, v, do, scale, causal)
    it = BW.intermediates(q, k, v, do, scale, causal)
    p, dp, delta, ds = it["P"], it["dP"], it["delta"], it["dS"]
    fin = np.isfinite(lse_ref)
    eps = np.where(fin, np.abs(np.where(fin, lse_gpu - lse_ref, 0.0)) + 2.0 ** -20 * (2 + np.abs(np.where(fin, lse_ref, 0.0))), 0.0)
    d = q.shape[-1]
    ddelta = (np.abs(do) * np.abs(o_gpu - o_ref)).sum(-1) + d * 2.0 ** -24 * (np.abs(do) * np.abs(o_ref)).sum(-1)
    tr = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
    b_dv = np.matmul(tr(p * (u + eps[..., None])), np.abs(do)) + u * np.abs(dv)
    sub = 2.0 ** -25 if dtype == "f16" else 0.0
    dds = p * (eps[..., None] * np.abs(dp - delta[..., None]) + ddelta[..., None]) + u * np.abs(ds) + sub
    b_dq = scale * np.matmul(dds, np.abs(k)) + u * np.abs(dq)
    b_dk = scale * np.matmul(tr(dds), np.abs(q)) + u * np.abs(dk)
    return (dq, dk, dv), (b_dq, b_dk, b_dv)


def check_grads(got, ref, bnd, what):
    ratios = []
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bnd):
        assert g.shape == r.shape, f"{what} {name}: shape {g.shape} vs {r.shape}"
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite values"
        if g.size == 0:
            continue
        err = np.abs(g - r)
        allow = 2.0 * b + 1e-6 * np.abs(r).max(initial=0.0)
        ratio = err / np.maximum(allow, 1e-300)
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        ratios.append(f"{name} {ratio[i]:.3f}")
        assert ratio[i] <= 1.0, (f"{what} {name}: |err| {err[i]:.3e} at {i} exceeds the bound {allow[i]:.3e} "
                                 f"(ref {r[i]:.4e}, max |err| {err.max():.3e})")
    print(f"{what}: max err/bound " + ", ".join(ratios))


CASES = [
    # B, H, Nq, Nk, d, dtype, causal
    (1, 2, 256, 256, 64, "f16", False),
    (2, 2, 300, 300, 128, "bf16", False),
    (1, 3, 520, 520, 128, "bf16", True),
    (1, 2, 200, 333, 64, "bf16", True),
    (1, 2, 333, 200, 128, "f16", True),
    (2, 1, 33, 1000, 128, "bf16", False),
    (1, 2, 1000, 40, 64, "f16", False),
    (1, 1, 1, 1, 64, "bf16", False),
    (1, 2, 129, 127, 128, "bf16", True),
    (1, 1, 640, 640, 64, "bf16", True),
    (1, 2, 300, 300, 256, "bf16", False),
    (1, 2, 333, 200, 256, "f16", True),
    (2, 1, 129, 520, 256, "bf16", True),
]


@pytest.mark.parametrize("B,H,nq,nk,d,dtype,causal", CASES)
def test_backward_vs_oracle(gpu_lib, B, H, nq, nk, d, dtype, causal):
    (qd, q), (kd, k), (vd, v), (dod, do) = _inputs(B, H, nq, nk, d, dtype, seed=nq * 7 + nk + d)
    scale = 1.0 / np.sqrt(d)
    what = f"bwd {B}x{H}x{nq}x{nk} d{d} {dtype} causal={causal}"
    print(what, flush=True)
    o, lse, dq, dk, dv = _gpu(gpu_lib, qd, kd, vd, dod, scale, causal)
    ref, bnd = bounds(q, k, v, do, o, lse, scale, causal, dtype)
    check_grads((dq, dk, dv), ref, bnd, what)


def test_backward_delta_workspace(gpu_lib):
    """The workspace holds rowsum(dO * O) of the O passed in."""
    (qd, q), (kd, k), (vd, v), (dod, do) = _inputs(1, 2, 150, 90, 64, "bf16", seed=4)
    o, lse = gpu_lib.forward(qd, kd, vd)
    delta = torch.empty((1, 2, 150), dtype=torch.float32, device="cuda")
    gpu_lib.backward(qd, kd, vd, o, lse, dod, delta=delta)
    torch.cuda.synchronize()
    ref = BW.row_delta(o.double().cpu().numpy(), do)
    got = delta.double().cpu().numpy()
    # fp32 sum of 64 exact products
    assert np.all(np.abs(got - ref) <= 64 * 2.0 ** -24 * (np.abs(do) * np.abs(o.double().cpu().numpy())).sum(-1) + 1e-30)


def test_backward_empty_sides(gpu_lib):
    """No keys: dQ = 0.  No queries: dK = dV = 0."""
    q = torch.randn((1, 2, 70, 128), device="cuda").to(torch.bfloat16)
    z = torch.zeros((1, 2, 0, 128), device="cuda", dtype=torch.bfloat16)
    o, lse = gpu_lib.forward(q, z, z)
    dq = torch.full_like(q, 7.0)
    gpu_lib.backward(q, z, z, o, lse, torch.randn_like(q), dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    k = torch.randn((1, 2, 90, 128), device="cuda").to(torch.bfloat16)
    qz = torch.zeros((1, 2, 0, 128), device="cuda", dtype=torch.bfloat16)
    lz = torch.zeros((1, 2, 0), device="cuda", dtype=torch.float32)
    dk = torch.full_like(k, 3.0)
    dv = torch.full_like(k, 3.0)
    gpu_lib.backward(qz, k, k, qz, lz, qz, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_deterministic(gpu_lib):
    (qd, _), (kd, _), (vd, _), (dod, _) = _inputs(1, 4, 700, 700, 128, "bf16", seed=9)
    o, lse = gpu_lib.forward(qd, kd, vd, causal=True)
    a = gpu_lib.backward(qd, kd, vd, o, lse, dod, causal=True)
    b = gpu_lib.backward(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_size(gpu_lib, causal):
    """The dense bf16 shape B=2 H=16 N=4096 d=128: two whole heads checked
    against the oracle (the launch covers all 32)."""
    w = W.WORKLOADS["dense_bf16"]
    rng = np.random.default_rng(11 + causal)
    shape = (w.B, w.H, w.Nq, w.d)
    (qd, _), (kd, _), (vd, _), (dod, _) = (to_device(rng.standard_normal(shape, dtype=np.float32), "bf16")
                                           for _ in range(4))
    o, lse = gpu_lib.forward(qd, kd, vd, causal=causal, scale=w.scale)
    dq, dk, dv = gpu_lib.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 15)):
        f = lambda t: t[b, h].double().cpu().numpy()  # noqa: E731
        ref, bnd = bounds(f(qd), f(kd), f(vd), f(dod), f(o), f(lse), w.scale, causal, "bf16")
        check_grads((f(dq), f(dk), f(dv)), ref, bnd, f"full-size bwd head ({b},{h}) causal={causal}")


# more sequences than a wave's 64 lanes: the kernels' slot lookup first picks
# a block of 64 sequences
MANY_Q = [int(x) for x in np.random.default_rng(11).integers(0, 150, 90)] + [0, 1, 64]
MANY_K = [int(x) for x in np.random.default_rng(12).integers(0, 150, 90)] + [3, 0, 64]

VARLEN_CASES = [
    # H, q lengths, k lengths, d, dtype, causal
    (1, MANY_Q, MANY_Q, 64, "bf16", True),
    (1, MANY_Q, MANY_K, 128, "bf16", False),
    (2, [300, 129, 64, 1], [300, 129, 64, 1], 128, "bf16", True),
    (3, [200, 0, 77], [150, 40, 300], 64, "f16", False),
    (2, [513, 260], [513, 260], 64, "bf16", True),
    (2, [100, 33, 250], [90, 0, 250], 128, "bf16", False),
    (2, [300, 129, 1], [300, 129, 1], 256, "bf16", True),
]


@pytest.mark.parametrize("H,lq,lk,d,dtype,causal", VARLEN_CASES)
def test_backward_varlen_vs_oracle(gpu_lib, H, lq, lk, d, dtype, causal):
    """Packed sequences ([H, T, d] with cu_seqlens): every sequence checked
    against the oracle's gradients of that sequence alone, to the same
    element-wise bound; sequences with no queries get dK = dV = 0, with no
    keys dQ = 0."""
    rng = np.random.default_rng(sum(lq) + d)
    cu_q, cu_k = np.cumsum([0] + lq).astype(np.int32), np.cumsum([0] + lk).astype(np.int32)
    (qd, q), (dod, do) = (to_device(rng.standard_normal((H, cu_q[-1], d), dtype=np.float32), dtype) for _ in range(2))
    (kd, k), (vd, v) = (to_device(rng.standard_normal((H, cu_k[-1], d), dtype=np.float32), dtype) for _ in range(2))
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward(qd, kd, vd, causal=causal, scale=scale, cu_seqlens_q=cq, cu_seqlens_k=ck)
    dq, dk, dv = gpu_lib.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, cu_seqlens_q=cq,
                                  cu_seqlens_k=ck)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()  # noqa: E731
    o, lse, dq, dk, dv = f(o), f(lse), f(dq), f(dk), f(dv)
    what = f"varlen bwd H{H} lq{lq[:8]} ({len(lq)} sequences) lk{lk[:8]} d{d} {dtype} causal={causal}"
    print(what, flush=True)
    for s in range(len(lq)):
        sq, sk = slice(cu_q[s], cu_q[s + 1]), slice(cu_k[s], cu_k[s + 1])
        if lq[s] == 0:
            assert np.all(dk[:, sk] == 0.0) and np.all(dv[:, sk] == 0.0)
            continue
        if lk[s] == 0:
            assert np.all(dq[:, sq] == 0.0)
            continue
        ref, bnd = bounds(q[:, sq], k[:, sk], v[:, sk], do[:, sq], o[:, sq], lse[:, sq], scale, causal, dtype)
        check_grads((dq[:, sq], dk[:, sk], dv[:, sk]), ref, bnd, f"{what} seq {s}")


def test_backward_key_offsets_beyond_2_31(gpu_lib):
    """K, V, dK and dV of more than 2^31 elements (B1 H3, 77 queries, Nk =
    4099 * 2047, d = 128: head 2 starts past element 2^31).  Key j of head h
    is row j mod 4099 of that head's seeded bank (K and V alike), so each
    (key, value) pair appears m = 2047 times.  Each copy then takes 1/m of
    the pair's softmax weight: dQ equals dQ of the bank problem, and dK and
    dV of every copy are the bank problem's dK and dV over m (the forward's
    lse is ln m above the bank's).  dQ is checked on every row, dK and dV on
    sampled copies, with the bounds above scaled the same way."""
    H, nq, d, R, m = 3, 77, 128, 4099, 2047
    nk = R * m
    (qd, q), (kbd, kb), (vbd, vb), (dod, do) = _inputs(1, H, nq, R, d, "bf16", seed=99)
    idx = torch.arange(nk, dtype=torch.int64, device="cuda") % R
    kd = kbd[0].index_select(1, idx).view(1, H, nk, d)
    vd = vbd[0].index_select(1, idx).view(1, H, nk, d)
    del idx
    assert kd.stride(1) * 2 > 2 ** 31
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward(qd, kd, vd, scale=scale)
    dq, dk, dv = gpu_lib.backward(qd, kd, vd, o, lse, dod, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    js = np.unique(np.concatenate([[0, 1, R - 1, R, nk // 2, nk - 2, nk - 1], rng.integers(0, nk, 40)]))
    jt = torch.from_numpy(js).cuda()
    f = lambda t: t.double().cpu().numpy()  # noqa: E731
    dk_s = f(dk.view(H, nk, d).index_select(1, jt))[None]
    dv_s = f(dv.view(H, nk, d).index_select(1, jt))[None]
    o_n, lse_n, dq_n = f(o), f(lse), f(dq)
    del kd, vd, dk, dv
    torch.cuda.empty_cache()
    (rq, rk, rv), (bq, bk, bv) = bounds(q, kb, vb, do, o_n, lse_n - np.log(m), scale, False, "bf16")
    r = js % R
    check_grads((dq_n, dk_s, dv_s), (rq, rk[:, :, r] / m, rv[:, :, r] / m), (bq, bk[:, :, r] / m, bv[:, :, r] / m),
                "bwd offsets beyond 2^31")
