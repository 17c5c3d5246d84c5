"""GPU parity of the fp16/bf16 attention kernels against the fp64 oracle.

Inputs are seeded N(0,1) (workloads.py), rounded to fp16/bf16; the oracle
sees the exact rounded values.  Bars: max |O - O_ref| <= 2e-3 (fp16) /
8e-3 (bf16) on every element; |lse - lse_ref| <= 1e-3 max(1, |lse_ref|).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import exact as OX
import workloads as W
from gpu_util import check, run_dense, sample_rows, to_device

pytestmark = pytest.mark.gpu


def test_tiny_config(gpu_lib):
    """1 x 2 heads, 256 x 256, d 64, fp16, non-causal, seed 0."""
    w = W.WORKLOADS["tiny_f16"]
    x = W.make_inputs(w)
    o, lse, (q, k, v, s) = run_dense(gpu_lib, x["q"], x["k"], x["v"], "f16", False)
    assert o.shape == (1, 2, 256, 64) and lse.shape == (1, 2, 256)
    o_ref, l_ref = oracle.attention(q, k, v, s, False)
    check(o, lse, o_ref, l_ref, "f16", "tiny")


SHAPES = [(1, 1), (17, 17), (127, 127), (128, 128), (129, 129), (300, 1000), (1000, 300), (257, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_dense_sweep(gpu_lib, dtype, d, causal, nq, nk):
    q, k, v = W.random_problem(1, 2, nq, nk, d, seed=nq * 7 + nk + d)
    k, v = k[:, :, :nk], v[:, :, :nk]
    o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, dtype, causal)
    o_ref, l_ref = oracle.attention(q64, k64, v64, s, causal)
    check(o, lse, o_ref, l_ref, dtype, f"{dtype} d{d} causal{causal} {nq}x{nk}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_batch_heads_and_scale(gpu_lib, dtype):
    """B > 1, H > 1, a non-default scale: heads must not mix."""
    q, k, v = W.random_problem(3, 5, 200, 333, 128, seed=5)
    for causal in (False, True):
        o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, dtype, causal, scale=0.21)
        o_ref, l_ref = oracle.attention(q64, k64, v64, s, causal)
        check(o, lse, o_ref, l_ref, dtype, f"B3H5 causal{causal}")


def test_empty_keys(gpu_lib):
    """Nk = 0: O = 0 and lse = -inf, no NaN."""
    q, _, _ = W.random_problem(1, 2, 70, 1, 64, seed=3)
    qd, _ = to_device(q, "bf16")
    kd = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = gpu_lib.forward(qd, kd, kd, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_zero_scale_uniform(gpu_lib):
    """scale = 0: uniform weights over the visible keys (mean / prefix mean)."""
    q, k, v = W.random_problem(1, 1, 150, 150, 64, seed=4)
    for causal in (False, True):
        o, lse, (q64, k64, v64, _) = run_dense(gpu_lib, q, k, v, "f16", causal, scale=0.0)
        o_ref, l_ref = oracle.attention(q64, k64, v64, 0.0, causal)
        check(o, lse, o_ref, l_ref, "f16", f"scale0 causal{causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_identical_keys_closed_form(gpu_lib, dtype):
    """All keys equal: O = mean of V (causal: prefix mean), lse = s_i + ln(count)."""
    nq = nk = 300
    d = 128
    q, _, v = W.random_problem(1, 1, nq, nk, d, seed=8)
    k = np.repeat(W.random_problem(1, 1, 1, 1, d, seed=9)[1], nk, axis=2)
    for causal in (False, True):
        o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, dtype, causal)
        s_i = s * (q64[0, 0] @ k64[0, 0, 0])
        if causal:
            ref = np.cumsum(v64[0, 0], axis=0) / np.arange(1, nk + 1)[:, None]
            lref = s_i + np.log(np.arange(1, nq + 1))
        else:
            ref = np.broadcast_to(v64[0, 0].mean(0), (nq, d))
            lref = s_i + np.log(nk)
        check(o[0, 0], lse[0, 0], ref, lref, dtype, f"identical keys causal{causal}")


def test_causal_row0_exact(gpu_lib):
    """Causal row 0 sees only key 0: O_0 = V_0 exactly (the weights are normalised by their own sum)."""
    q, k, v = W.random_problem(2, 3, 129, 129, 128, seed=12)
    v[..., 0, :] *= 3.0  # large |V_0|: a bf16 relative error would show
    o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, "bf16", True)
    assert np.array_equal(o[:, :, 0], v64[:, :, 0])


def test_determinism_and_canaries(gpu_lib):
    """Two runs are bitwise equal; guard regions around O and lse stay untouched."""
    q, k, v = W.random_problem(2, 4, 333, 517, 128, seed=21)
    qd, _ = to_device(q, "bf16")
    kd, _ = to_device(k, "bf16")
    vd, _ = to_device(v, "bf16")
    guard = 4096
    n_o, n_l = qd.numel(), 2 * 4 * 333
    for causal in (False, True):
        outs = []
        for _ in range(2):
            ob = torch.full((n_o + 2 * guard,), 12345.0, dtype=torch.bfloat16, device="cuda")
            lb = torch.full((n_l + 2 * guard,), -7.0, dtype=torch.float32, device="cuda")
            o = ob[guard:guard + n_o].view(qd.shape)
            lse = lb[guard:guard + n_l].view(2, 4, 333)
            gpu_lib.forward(qd, kd, vd, causal=causal, out=o, lse=lse)
            torch.cuda.synchronize()
            assert torch.all(ob[:guard] == 12345.0) and torch.all(ob[guard + n_o:] == 12345.0)
            assert torch.all(lb[:guard] == -7.0) and torch.all(lb[guard + n_l:] == -7.0)
            outs.append((o.clone(), lse.clone()))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------- varlen

def run_varlen(attn, lengths_q, lengths_k, H, d, dtype, causal, seed):
    cq, ck = W.cu_seqlens(lengths_q), W.cu_seqlens(lengths_k)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, int(cq[-1]), d), dtype=np.float32)
    k = rng.standard_normal((H, int(ck[-1]), d), dtype=np.float32)
    v = rng.standard_normal((H, int(ck[-1]), d), dtype=np.float32)
    qd, q64 = to_device(q, dtype)
    kd, k64 = to_device(k, dtype)
    vd, v64 = to_device(v, dtype)
    s = 1.0 / np.sqrt(d)
    o, lse = attn.forward(qd, kd, vd, causal=causal, scale=s,
                          cu_seqlens_q=torch.from_numpy(cq).cuda(), cu_seqlens_k=torch.from_numpy(ck).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q64, k64, v64, cq, ck, s, causal)
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen(gpu_lib, dtype, causal, d):
    lengths = [1, 0, 127, 129, 2048, 300]
    o, lse, o_ref, l_ref = run_varlen(gpu_lib, lengths, lengths, 2, d, dtype, causal, seed=d)
    check(o, lse, o_ref, l_ref, dtype, f"varlen {dtype} d{d} causal{causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,nseq", [(64, 150), (128, 150), (128, 36), (256, 40)])
def test_varlen_many_sequences_every_row_written(gpu_lib, causal, d, nseq):
    """More sequences than the kernels' scalar lookup takes (16) and than one
    wave's 64 lanes (the lookup then picks a block of 64 first): empty,
    one-token and ragged sequences, query and key lengths that differ.  O
    and lse start as NaN, so that a work item the lookup skipped shows up."""
    lq = [int(x) for x in np.random.default_rng(7).integers(0, 400, nseq)] + [0, 1, 128, 129]
    lk = [int(x) for x in np.random.default_rng(8).integers(0, 400, nseq)] + [3, 0, 128, 1]
    cq, ck = W.cu_seqlens(lq), W.cu_seqlens(lk)
    H = 3
    rng = np.random.default_rng(d + causal)
    qd, q64 = to_device(rng.standard_normal((H, int(cq[-1]), d), dtype=np.float32), "bf16")
    kd, k64 = to_device(rng.standard_normal((H, int(ck[-1]), d), dtype=np.float32), "bf16")
    vd, v64 = to_device(rng.standard_normal((H, int(ck[-1]), d), dtype=np.float32), "bf16")
    o = torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(qd.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    s = 1.0 / np.sqrt(d)
    gpu_lib.forward(qd, kd, vd, causal=causal, scale=s, cu_seqlens_q=torch.from_numpy(cq).cuda(),
                    cu_seqlens_k=torch.from_numpy(ck).cuda(), out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q64, k64, v64, cq, ck, s, causal)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref, "bf16",
          f"varlen {len(lq)} sequences d{d} causal{causal}")


def test_varlen_persistent_grid_streams_and_graph(gpu_lib):
    """Past 16 sequences a packed batch runs on a persistent grid whose work
    queues are kept per stream and cleared by each launch's last workgroup:
    repeated launches, launches on two streams at once and the replays of a
    captured graph (whose launch takes the dispatcher) all give bitwise the
    O and lse of the first launch, which matches the oracle."""
    lq = [int(x) for x in np.random.default_rng(11).integers(0, 300, 40)] + [0, 1]
    cq = W.cu_seqlens(lq)
    H, d, s = 4, 64, 0.125
    rng = np.random.default_rng(12)
    (qd, q64), (kd, k64), (vd, v64) = (to_device(rng.standard_normal((H, int(cq[-1]), d), dtype=np.float32), "bf16")
                                       for _ in range(3))
    cu = torch.from_numpy(cq).cuda()

    def run(o, lse):
        gpu_lib.forward(qd, kd, vd, causal=True, scale=s, cu_seqlens_q=cu, cu_seqlens_k=cu, out=o, lse=lse)

    def fresh():
        return (torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device="cuda"),
                torch.full(qd.shape[:2], float("nan"), dtype=torch.float32, device="cuda"))

    o0, l0 = fresh()
    run(o0, l0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q64, k64, v64, cq, cq, s, True)
    check(o0.double().cpu().numpy(), l0.double().cpu().numpy(), o_ref, l_ref, "bf16", "persistent grid")
    for _ in range(3):
        o, lse = fresh()
        run(o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(lse, l0)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        outs = [fresh() for _ in streams]
        torch.cuda.synchronize()
        for st, (o, lse) in zip(streams, outs):
            with torch.cuda.stream(st):
                run(o, lse)
        torch.cuda.synchronize()
        for o, lse in outs:
            assert torch.equal(o, o0) and torch.equal(lse, l0)
    og, lg = fresh()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run(og, lg)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(og, lg)
    for _ in range(3):
        og.fill_(float("nan"))
        lg.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(og, o0) and torch.equal(lg, l0)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_q_k_lengths_differ(gpu_lib, causal):
    """Per-sequence Nq_b != Nk_b, including an empty key sequence (O = 0, lse = -inf)."""
    lq = [5, 130, 64, 200, 33]
    lk = [9, 100, 0, 260, 33]
    o, lse, o_ref, l_ref = run_varlen(gpu_lib, lq, lk, 3, 128, "bf16", causal, seed=77)
    check(o, lse, o_ref, l_ref, "bf16", f"varlen q!=k causal{causal}")


# ---------------------------------------------------------------- full sizes (sampled rows)

FULL = ["dense_bf16", "dense_bf16_causal", "hdim256_bf16", "n8k_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(gpu_lib, name):
    """The benchmark shapes in the benchmark's launch configuration; the oracle
    checks sampled rows of sampled heads (it cannot materialise all of S)."""
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, x["q"], x["k"], x["v"], w.dtype, w.causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(1)
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [tuple(rng.integers(0, [w.B, w.H])) for _ in range(2)]
    for (b, h) in heads:
        rows = sample_rows(w.Nq, 48, seed=b * 100 + h)
        o_ref, l_ref = OX.attention_rows(q64[b, h], k64[b, h], v64[b, h], rows, s, w.causal)
        check(o[b, h][rows], lse[b, h][rows], o_ref, l_ref, w.dtype, f"{name} b{b} h{h}")


def test_full_size_varlen_sampled(gpu_lib):
    w = W.WORKLOADS["varlen_bf16_causal"]
    x = W.make_inputs(w)
    cu = x["cu_seqlens"]
    qd, q64 = to_device(x["q"], "bf16")
    kd, k64 = to_device(x["k"], "bf16")
    vd, v64 = to_device(x["v"], "bf16")
    cud = torch.from_numpy(cu).cuda()
    o, lse = gpu_lib.forward(qd, kd, vd, causal=True, scale=w.scale, cu_seqlens_q=cud, cu_seqlens_k=cud)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for h in (0, w.H - 1, 13):
        for b in range(w.B):
            a, e = int(cu[b]), int(cu[b + 1])
            rows = sample_rows(e - a, 8, seed=b + h)
            o_ref, l_ref = OX.attention_rows(q64[h, a:e], k64[h, a:e], v64[h, a:e], rows, w.scale, True)
            check(o[h, a:e][rows], lse[h, a:e][rows], o_ref, l_ref, "bf16", f"varlen full h{h} seq{b}")


def test_query_tile_pair_paths(gpu_lib):
    """Dense launches may run two query tiles per workgroup: across heads h
    and h + heads/2 when the head count is even (the full-size tests), within
    one head (t, T-1-t) when it is odd.  Odd head counts: causal (always
    paired) on the whole output, and non-causal with enough tiles for pairs
    to cover every CU (B1 H5 N=26624: 5 x 52 pairs) on sampled rows of
    every head, including the middle tile of an odd tile count."""
    q, k, v = W.random_problem(1, 3, 1000, 1000, 128, seed=77)
    o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, "bf16", True)
    o_ref, l_ref = oracle.attention(q64, k64, v64, s, True)
    check(o, lse, o_ref, l_ref, "bf16", "causal, 3 heads")

    n = 26624 - 256  # 103 tiles of 256 rows: an odd count, the middle tile alone
    q, k, v = W.random_problem(1, 5, n, n, 128, seed=78)
    o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, "bf16", False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    mid = 51 * 256
    for h in range(5):
        rows = np.unique(np.concatenate([sample_rows(n, 24, seed=h), [mid, mid + 255]]))
        o_ref, l_ref = OX.attention_rows(q64[0, h], k64[0, h], v64[0, h], rows, s, False)
        check(o[0, h][rows], lse[0, h][rows], o_ref, l_ref, "bf16", f"non-causal paired, head {h}")


@pytest.mark.parametrize("causal", [False, True])
def test_offsets_beyond_2_31_elements(gpu_lib, causal):
    """Q and O of more than 2^31 elements (B1 H3, Nq = 2^23 + 37, d = 128:
    head 2 starts at element 2^31 + 9472, byte 2^32 + 18944) against 64 keys,
    so the 64-bit row offsets of the loads and of the O and lse stores are
    exercised at a cost of a few milliseconds.  Q row g (g = head * Nq + i)
    is row (g * 2654435761 + 12345) mod 4096 of a seeded N(0,1) bank,
    gathered on the device; the host recomputes the index for sampled rows.
    Rows >= 63 see all 64 keys, causal or not."""
    H, nq, nk, d, R = 3, 2 ** 23 + 37, 64, 128, 4096
    bank32, _, _ = W.random_problem(1, 1, R, 1, d, seed=91)
    _, k32, v32 = W.random_problem(1, H, 1, nk, d, seed=92)
    bank_d, bank64 = to_device(bank32[0, 0], "bf16")
    kd, k64 = to_device(k32, "bf16")
    vd, v64 = to_device(v32, "bf16")

    def bank_index(g):
        return (g * 2654435761 + 12345) % R

    g = torch.arange(H * nq, dtype=torch.int64, device="cuda")
    qd = bank_d.index_select(0, bank_index(g)).view(1, H, nq, d)
    del g
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert (int(qd.numel()) > 2 ** 31) and qd.stride(1) * 2 > 2 ** 31
    for h in range(H):
        rows = np.unique(np.concatenate([sample_rows(nq, 24, seed=h), np.arange(0, 64, 9), [nq - 1]]))
        ri = torch.from_numpy(rows).cuda()
        o_h = o[0, h].index_select(0, ri).double().cpu().numpy()
        l_h = lse[0, h].index_select(0, ri).double().cpu().numpy()
        q_rows = bank64[bank_index(np.int64(h) * nq + rows.astype(np.int64))]
        far = rows >= nk - 1
        o_ref = np.empty_like(o_h)
        l_ref = np.empty_like(l_h)
        o_ref[far], l_ref[far] = OX.attention_rows(q_rows[far], k64[0, h], v64[0, h], np.arange(far.sum()),
                                                   scale, False)
        if np.any(~far):
            q_head = bank64[bank_index(np.int64(h) * nq + np.arange(nk, dtype=np.int64))]
            o_ref[~far], l_ref[~far] = OX.attention_rows(q_head, k64[0, h], v64[0, h], rows[~far], scale, causal)
        check(o_h, l_h, o_ref, l_ref, "bf16", f"offsets beyond 2^31, head {h}, causal {causal}")
    del qd, o, lse
    torch.cuda.empty_cache()


def test_key_offsets_beyond_2_31_elements(gpu_lib):
    """K and V of more than 2^31 elements (B1 H3, Nk = 4099 * 2047 = 8390653,
    d = 128: head 2 starts past element 2^31 and byte 2^32; the last key tile
    holds 125 keys) for 77 queries, one pass and in 8 key chunks.  Key j of
    head h is row j mod 4099 of that head's seeded N(0,1) bank (K and V
    alike), so every (key, value) pair of the bank appears exactly m = 2047
    times.  Repeating each pair m times leaves the softmax average O
    unchanged and adds ln m to the logsumexp, so the oracle runs on the bank
    alone.  4099 is prime: an offset cut at 2^32 bytes (2^24 rows) lands on
    other rows, and the banks differ per head."""
    H, nq, d, R, m = 3, 77, 128, 4099, 2047
    nk = R * m
    q32, kb32, vb32 = W.random_problem(1, H, nq, R, d, seed=93)
    qd, q64 = to_device(q32, "bf16")
    kb_d, kb64 = to_device(kb32, "bf16")
    vb_d, vb64 = to_device(vb32, "bf16")
    idx = torch.arange(nk, dtype=torch.int64, device="cuda") % R
    kd = kb_d[0].index_select(1, idx).view(1, H, nk, d)
    vd = vb_d[0].index_select(1, idx).view(1, H, nk, d)
    del idx
    assert kd.stride(1) * 2 > 2 ** 31
    scale = 1.0 / np.sqrt(d)
    runs = {"one pass": gpu_lib.forward(qd, kd, vd, causal=False, scale=scale),
            "8 key chunks": gpu_lib.forward_splitkv(qd, kd, vd, causal=False, scale=scale, num_splits=8)}
    torch.cuda.synchronize()
    for what, (o, lse) in runs.items():
        o = o.double().cpu().numpy()
        lse = lse.double().cpu().numpy()
        for h in range(H):
            rows = np.arange(nq)
            o_ref, l_ref = OX.attention_rows(q64[0, h], kb64[0, h], vb64[0, h], rows, scale, False)
            check(o[0, h], lse[0, h], o_ref, l_ref + np.log(m), "bf16", f"{what}, head {h}")
    del qd, kd, vd, runs
    torch.cuda.empty_cache()


def test_varlen_offsets_beyond_2_31_elements(gpu_lib):
    """Packed batches whose rows of head 2 start past element 2^31, H3 d128.

    Non-causal, long keys: 2 sequences of 70 and 57 queries over 4099 * 1024
    and 4099 * 1023 keys; key g of sequence b is row g mod 4099 of that
    (head, sequence)'s bank, so O is attention over the bank and lse is ln m
    above it.  Causal, long queries: 2^22 + 37 and 2^22 + 11 queries over 64
    keys each (Q row g of the pack is row (g * 2654435761 + 12345) mod 4096 of
    a seeded bank); rows >= 63 of a sequence see all of its keys, rows below
    that are checked against the first 64 rows."""
    H, d, R = 3, 128, 4099
    scale = 1.0 / np.sqrt(d)
    # -- non-causal, long keys
    lq, ms = [70, 57], [1024, 1023]
    lk = [R * m for m in ms]
    tk = sum(lk)
    assert 2 * tk * d > 2 ** 31
    q32, _, _ = W.random_problem(1, H, sum(lq), 1, d, seed=31)
    qd, q64 = to_device(q32[0], "bf16")
    banks = [to_device(W.random_problem(1, H, 1, R, d, seed=32 + b)[1][0], "bf16") for b in range(4)]
    (kb0, k64_0), (kb1, k64_1), (vb0, v64_0), (vb1, v64_1) = banks
    kd = torch.cat([kb0.index_select(1, torch.arange(lk[0], device="cuda") % R),
                    kb1.index_select(1, torch.arange(lk[1], device="cuda") % R)], dim=1).contiguous()
    vd = torch.cat([vb0.index_select(1, torch.arange(lk[0], device="cuda") % R),
                    vb1.index_select(1, torch.arange(lk[1], device="cuda") % R)], dim=1).contiguous()
    cq = torch.tensor([0, lq[0], lq[0] + lq[1]], dtype=torch.int32, device="cuda")
    ck = torch.tensor([0, lk[0], tk], dtype=torch.int32, device="cuda")
    o, lse = gpu_lib.forward(qd, kd, vd, causal=False, scale=scale, cu_seqlens_q=cq, cu_seqlens_k=ck)
    torch.cuda.synchronize()
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    del kd, vd
    torch.cuda.empty_cache()
    for h in range(H):
        for b, (kb64, vb64) in enumerate([(k64_0, v64_0), (k64_1, v64_1)]):
            a = 0 if b == 0 else lq[0]
            rows = np.arange(lq[b])
            o_ref, l_ref = OX.attention_rows(q64[h, a:a + lq[b]], kb64[h], vb64[h], rows, scale, False)
            check(o[h, a:a + lq[b]], lse[h, a:a + lq[b]], o_ref, l_ref + np.log(ms[b]), "bf16",
                  f"varlen long keys, head {h}, seq {b}")
    # -- causal, long queries
    lq2, nk = [2 ** 22 + 37, 2 ** 22 + 11], 64
    tq = sum(lq2)
    assert 2 * tq * d > 2 ** 31
    bank32, _, _ = W.random_problem(1, 1, 4096, 1, d, seed=41)
    _, k32, v32 = W.random_problem(1, H, 1, 2 * nk, d, seed=42)
    bank_d, bank64 = to_device(bank32[0, 0], "bf16")
    kd, k64 = to_device(k32[0], "bf16")
    vd, v64 = to_device(v32[0], "bf16")

    def bank_index(g):
        return (g * 2654435761 + 12345) % 4096

    g = torch.arange(H * tq, dtype=torch.int64, device="cuda")
    qd = bank_d.index_select(0, bank_index(g)).view(H, tq, d)
    del g
    cq = torch.tensor([0, lq2[0], tq], dtype=torch.int32, device="cuda")
    ck = torch.tensor([0, nk, 2 * nk], dtype=torch.int32, device="cuda")
    o, lse = gpu_lib.forward(qd, kd, vd, causal=True, scale=scale, cu_seqlens_q=cq, cu_seqlens_k=ck)
    torch.cuda.synchronize()
    for h in range(H):
        for b in range(2):
            a = 0 if b == 0 else lq2[0]
            rows = np.unique(np.concatenate([sample_rows(lq2[b], 16, seed=h + 3 * b), np.arange(0, 64, 9)]))
            ri = torch.from_numpy(a + rows).cuda()
            o_h = o[h].index_select(0, ri).double().cpu().numpy()
            l_h = lse[h].index_select(0, ri).double().cpu().numpy()
            ks, vs = k64[h, b * nk:(b + 1) * nk], v64[h, b * nk:(b + 1) * nk]
            far = rows >= nk - 1
            o_ref, l_ref = np.empty_like(o_h), np.empty_like(l_h)
            qf = bank64[bank_index(np.int64(h) * tq + a + rows[far].astype(np.int64))]
            o_ref[far], l_ref[far] = OX.attention_rows(qf, ks, vs, np.arange(far.sum()), scale, False)
            if np.any(~far):
                q0 = bank64[bank_index(np.int64(h) * tq + a + np.arange(nk, dtype=np.int64))]
                o_ref[~far], l_ref[~far] = OX.attention_rows(q0, ks, vs, rows[~far], scale, True)
            check(o_h, l_h, o_ref, l_ref, "bf16", f"varlen long queries causal, head {h}, seq {b}")
    del qd, o, lse
    torch.cuda.empty_cache()


DRIFT_SHAPES = ["rising", "falling", "spiky", "partial"]


def _drift_problem(nq, nk, d, shape, seed, heads=2):
    """Score rows whose maximum drifts across key tiles.  Channel 0 of every
    query is 1 and channel 0 of key j is a ramp, so each row's scores climb
    (or fall) by about 0.03 in base 2 per key: several bits per key tile, with
    a jump of 20 at key 700 on the rising ramp.  The running max then moves on
    most tiles, the reference of the exponentials lags it, and P can exceed
    1 (up to the kernel's slack) before a rescale; the other channels are
    small N(0,1) noise.  "spiky": one key per 128 keys (index 37 mod 128)
    stands 3 more bits above the previous one and the rest 40 below, so the
    weight of a row sits on about one key while the reference lags the row
    max by up to 3 bits; V is then uniform in (-3.9, 3.9), so many |O| lie in
    [2, 4): there the output rounding alone takes up to half an ulp of the
    bar, and P rounded to 16 bits would add up to 2^-9 |V| in bf16 unless the
    kernel takes its residual pass.  "partial": the rising ramp reaches only
    every third query row (the others see the noise alone), so one row's
    trigger moves the reference of rows that lag it by less than the slack.
    Returns fp32 q [1, heads, nq, d], k, v [1, heads, nk, d]."""
    rng = np.random.default_rng(seed)
    q = 0.1 * rng.standard_normal((1, heads, nq, d)).astype(np.float32)
    k = 0.1 * rng.standard_normal((1, heads, nk, d)).astype(np.float32)
    v = rng.standard_normal((1, heads, nk, d)).astype(np.float32)
    q[..., 0] = 1.0
    step = 0.03 / (np.log2(np.e) / np.sqrt(d))  # base-2 increase per key
    ramp = step * np.arange(nk, dtype=np.float64)
    if shape in ("rising", "partial"):
        ramp[700:] += 20.0 / (np.log2(np.e) / np.sqrt(d))
        if shape == "partial":
            q[..., np.arange(nq) % 3 != 0, 0] = 0.0
    elif shape == "falling":
        ramp = ramp[::-1].copy()
    else:
        j = np.arange(nk)
        bits = np.where(j % 128 == 37, 3.0 * (j // 128), -40.0)
        ramp = bits / (np.log2(np.e) / np.sqrt(d))
        v[:] = rng.uniform(-3.9, 3.9, v.shape)
    k[..., 0] = ramp.astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", DRIFT_SHAPES)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_drifting_row_max(gpu_lib, dtype, causal, shape, d):
    """Drifting row maxima (``_drift_problem``) through the dense launches,
    Nk = 1000 (a ragged last tile): d = 64 and 128 at two waves per SIMD,
    d = 256 with its 64-key tiles at one wave per SIMD and late tile loads."""
    q, k, v = _drift_problem(300, 1000, d, shape, seed=5 + d)
    o, lse, (q64, k64, v64, s) = run_dense(gpu_lib, q, k, v, dtype, causal)
    o_ref, l_ref = oracle.attention(q64, k64, v64, s, causal)
    check(o, lse, o_ref, l_ref, dtype, f"drifting max {shape} d{d} causal{causal}")


@pytest.mark.parametrize("shape", DRIFT_SHAPES)
@pytest.mark.parametrize("d", [128, 256])
def test_drifting_row_max_varlen_causal(gpu_lib, shape, d):
    """The same rows packed as a variable-length causal batch of two
    sequences (1000 and 345 tokens, the second with its own ramp): at d = 128
    the 4-wave, 64-key tile configuration with late loads."""
    qa, ka, va = _drift_problem(1000, 1000, d, shape, seed=11 + d)
    qb, kb, vb = _drift_problem(345, 345, d, shape, seed=12 + d)
    cu = np.array([0, 1000, 1345], dtype=np.int32)
    q = np.concatenate([qa[0], qb[0]], axis=1)
    k = np.concatenate([ka[0], kb[0]], axis=1)
    v = np.concatenate([va[0], vb[0]], axis=1)
    qd, q64 = to_device(q, "bf16")
    kd, k64 = to_device(k, "bf16")
    vd, v64 = to_device(v, "bf16")
    cud = torch.from_numpy(cu).cuda()
    s = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward(qd, kd, vd, causal=True, scale=s, cu_seqlens_q=cud, cu_seqlens_k=cud)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q64, k64, v64, cu, cu, s, True)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref, "bf16",
          f"drifting max varlen causal {shape} d{d}")


@pytest.mark.parametrize("shape", DRIFT_SHAPES)
@pytest.mark.parametrize("d,causal,nq", [(128, False, 300), (128, True, 300), (256, False, 300), (128, False, 1),
                                         (256, False, 2), (64, True, 2)])
def test_drifting_row_max_splitkv(gpu_lib, shape, d, causal, nq):
    """Drifting maxima through the key-chunk launches (3 chunks of 334 keys:
    the ramp's maximum moves inside every chunk) and the merge; one or two
    query rows run the decoding-shaped kernel, whose lanes keep their own
    lazy reference max."""
    q, k, v = _drift_problem(nq, 1000, d, shape, seed=21 + d)
    qd, q64 = to_device(q, "bf16")
    kd, k64 = to_device(k, "bf16")
    vd, v64 = to_device(v, "bf16")
    s = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward_splitkv(qd, kd, vd, causal=causal, scale=s, num_splits=3)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q64, k64, v64, s, causal)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref, "bf16",
          f"drifting max split-KV {shape} d{d} causal{causal} nq{nq}")


@pytest.mark.parametrize("shape", DRIFT_SHAPES)
@pytest.mark.parametrize("nq", [7, 1])
def test_drifting_row_max_paged_e4m3(gpu_lib, shape, nq):
    """Drifting maxima read from a paged e4m3 cache with per-(token, head)
    scales (64-token pages in shuffled order, d = 128, 7 queries).  Key j's
    channel 0 holds the code +-448 and its scale is |ramp_j| / 448, so the
    dequantised channel 0 is the ramp; the other channels are codes of
    magnitude <= 2 times that scale.  V: codes in [2, 3.75] with scales in
    [0.5, 1], so |V| reaches [2, 3.75] (spiky rows then have |O| in [2, 4)),
    and P, up to the slack's 16, is multiplied by the V scale before the
    16-bit packing."""
    from oracle import fp8 as F
    from oracle import paged as PG

    d, nk, H, P = 128, 1000, 2, 64  # one query row: the decoding-shaped kernel
    q, k, _ = _drift_problem(nq, nk, d, shape, seed=31, heads=H)
    rng = np.random.default_rng(33)
    ramp = k[0, :, :, 0].astype(np.float64)  # [H, nk]
    small = F.e4m3_encode(rng.choice([-2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0], (H, nk, d)))
    kcode = small.copy()
    kcode[..., 0] = F.e4m3_encode(np.where(ramp < 0, -448.0, 448.0))
    ksc = np.maximum(np.abs(ramp) / 448.0, 1e-6).astype(np.float32)
    vcode = F.e4m3_encode(rng.choice([2.0, 2.5, 3.0, 3.5, 3.75], (H, nk, d)) * rng.choice([-1.0, 1.0], (H, nk, d)))
    vsc = rng.uniform(0.5, 1.0, (H, nk)).astype(np.float32)
    n_pages = -(-nk // P) + 3
    perm = rng.permutation(n_pages)[: -(-nk // P)]
    kc = np.zeros((n_pages, P, H, d), np.uint8)
    vc = np.zeros((n_pages, P, H, d), np.uint8)
    ks = np.ones((n_pages, P, H), np.float32)
    vs = np.ones((n_pages, P, H), np.float32)
    for j, pg in enumerate(perm):
        rows = slice(j * P, min(nk, (j + 1) * P))
        n = rows.stop - rows.start
        kc[pg, :n] = np.transpose(kcode[:, rows], (1, 0, 2))
        vc[pg, :n] = np.transpose(vcode[:, rows], (1, 0, 2))
        ks[pg, :n] = ksc[:, rows].T
        vs[pg, :n] = vsc[:, rows].T
    table = perm.astype(np.int32)[None]
    qd, q64 = to_device(q, "bf16")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    s = 1.0 / np.sqrt(d)
    o, lse = gpu_lib.forward_paged(qd, t(kc), t(vc), t(table), torch.tensor([nk], dtype=torch.int32).cuda(),
                                   scale=s, k_scale=t(ks), v_scale=t(vs), kv_dtype="e4m3", num_splits=3)
    torch.cuda.synchronize()
    ref_o, ref_l = PG.attention_paged_quant(q64, kc, vc, ks, vs, table, np.array([nk]), s, "e4m3")
    kd = PG.dequantize(kc, ks, "e4m3")[perm[0], :5, 0, 0]
    assert np.allclose(kd, ramp[0, :5], rtol=1e-6, atol=1e-3)  # channel 0 carries the ramp
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, "bf16",
          f"drifting max paged e4m3 {shape} nq{nq}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_attn_fwd_null_stream(gpu_lib, dtype):
    """The entry point with the specified argument list, attn_fwd, which
    enqueues on the null stream (the other tests go through attn_fwd_stream
    on torch's current stream), called through the C ABI with raw pointers:
    bf16 and e4m3 codes, causal, B2 H3 Nq 300 Nk 700, against the oracle."""
    from oracle import fp8 as F

    B, H, nq, nk, d = 2, 3, 300, 700, 128
    scale = 0.09
    torch.cuda.synchronize()
    if dtype == "bf16":
        q, k, v = W.random_problem(B, H, nq, nk, d, seed=77)
        qd, q64 = to_device(q, "bf16")
        kd, k64 = to_device(k[:, :, :nk], "bf16")
        vd, v64 = to_device(v[:, :, :nk], "bf16")
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device="cuda")
        rc = gpu_lib.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, nq,
                              nk, d, scale, 1, None, None, gpu_lib.ATTN_DT_BF16, None, None, None)
        assert rc == gpu_lib.ATTN_OK
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q64, k64, v64, scale, True)
        check(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref, "bf16", "attn_fwd bf16")
    else:
        nt = lambda n: (n + 127) // 128  # noqa: E731
        codes = [0x38, 0x3C, 0x40, 0x44, 0x48, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8]
        q8 = W.random_codes_from(codes, (B, H, nq, d), 78)
        k8 = W.random_codes_from(codes, (B, H, nk, d), 79)
        v8 = W.random_codes_from(codes, (B, H, nk, d), 80)
        sq = W.random_pow2_scales((B, H, nt(nq)), 81, -1, 0)
        sk = W.random_pow2_scales((B, H, nt(nk)), 82, -1, 0)
        sv = W.random_pow2_scales((B, H, nt(nk)), 83, -7, -4)
        dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        tq, tk, tv, tsq, tsk, tsv = dv(q8), dv(k8), dv(v8), dv(sq), dv(sk), dv(sv)
        o = torch.full((B, H, nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device="cuda")
        rc = gpu_lib.attn_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, nq,
                              nk, d, scale, 1, None, None, gpu_lib.ATTN_DT_FP8_E4M3, tsq.data_ptr(), tsk.data_ptr(),
                              tsv.data_ptr())
        assert rc == gpu_lib.ATTN_OK
        torch.cuda.synchronize()
        ref = F.attention_fp8(q8, k8, v8, sq, sk, sv, scale, True, ambiguity=3e-5, parts=True)
        err = np.abs(o.double().cpu().numpy() - ref["o"]) - ref["flip"]
        # bf16 output rounding + fp32 accumulation (|O| < 0.5 here) and the
        # e4m3 MFMA's truncation of the PV sums (bounded as in test_gpu_fp8)
        from test_gpu_fp8 import _pv_bound

        assert np.all(err <= 4e-3 + _pv_bound(ref)), float(err.max())
        l = lse.double().cpu().numpy()
        assert np.all(np.abs(l - ref["lse"]) <= 1e-3 * np.maximum(1.0, np.abs(ref["lse"])))
