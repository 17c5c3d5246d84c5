"""GPU parity of attention over a paged key/value cache (attn_fwd_paged)
against ``oracle.paged`` (page-table gather, then the attention definition).

Caches are cut from dense per-sequence keys and values into pages stored in
a shuffled order, with noise in pages no sequence uses and garbage in the
page-table entries past each sequence's last page (never read).  Sequence
lengths are ragged (not multiples of the page size or the 64-key tile),
include an empty sequence, and the decoding shape (one query per head) is
checked in full.
"""

import numpy as np
import pytest
import torch

from oracle import paged as PG
from gpu_util import check, to_device

pytestmark = pytest.mark.gpu


def make_cache(B, H, lens, d, page_size, dtype, seed, spare=5):
    rng = np.random.default_rng(seed)
    max_pages = max(1, -(-max(lens) // page_size)) + 1  # one table column more than needed
    n_pages = B * max_pages + spare
    perm = rng.permutation(n_pages)
    kc = rng.standard_normal((n_pages, page_size, H, d), dtype=np.float32)
    vc = rng.standard_normal((n_pages, page_size, H, d), dtype=np.float32)
    table = np.full((B, max_pages), -7, dtype=np.int32)  # entries past a sequence's pages: garbage
    table[:, -1] = 10 ** 6
    for b in range(B):
        for j in range(-(-lens[b] // page_size)):
            table[b, j] = perm[b * max_pages + j]
    return kc, vc, table


def run_case(attn, B, H, Nq, d, dtype, page_size, lens, splits, seed):
    kc32, vc32, table = make_cache(B, H, lens, d, page_size, dtype, seed)
    rng = np.random.default_rng(seed + 1)
    qd, q = to_device(rng.standard_normal((B, H, Nq, d), dtype=np.float32), dtype)
    kcd, kc = to_device(kc32, dtype)
    vcd, vc = to_device(vc32, dtype)
    td = torch.from_numpy(table).cuda()
    sd = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(d)
    o, lse = attn.forward_paged(qd, kcd, vcd, td, sd, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = PG.attention_paged(q, kc, vc, table, np.array(lens), scale)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, dtype,
          f"paged B{B} H{H} Nq{Nq} d{d} P{page_size} lens{lens} S{splits}")


CASES = [
    # B, H, Nq, d, dtype, page_size, lens, splits
    (3, 4, 1, 128, "bf16", 64, [1000, 70, 513], 4),
    (2, 2, 1, 128, "f16", 128, [4096, 1], 8),
    (4, 2, 3, 64, "bf16", 64, [300, 0, 64, 129], 3),
    (2, 2, 1, 256, "bf16", 256, [2000, 777], 5),
    (1, 8, 130, 128, "bf16", 192, [900], 2),
    (2, 3, 1, 128, "bf16", 64, [63, 65], 1),
    (2, 2, 7, 64, "f16", 128, [5000, 2500], 16),
    (2, 2, 8, 128, "bf16", 64, [700, 1], 3),
    (1, 3, 2, 256, "f16", 64, [1111], 7),
]


@pytest.mark.parametrize("B,H,Nq,d,dtype,page_size,lens,splits", CASES)
def test_paged_vs_oracle(gpu_lib, B, H, Nq, d, dtype, page_size, lens, splits):
    run_case(gpu_lib, B, H, Nq, d, dtype, page_size, lens, splits, seed=sum(lens) + d)


def test_paged_decode_full(gpu_lib):
    """Decoding: B=8 sequences of up to 8192 cached tokens, H=32, d=128,
    256-token pages, default chunk count; every row checked."""
    lens = [8192, 5000, 1, 4097, 7777, 256, 3000, 6144]
    run_case(gpu_lib, 8, 32, 1, 128, "bf16", 256, lens, None, seed=12)


def test_paged_matches_contiguous_splitkv(gpu_lib):
    """One sequence per batch entry whose pages are in order: the paged
    launch reads the same rows as the contiguous split-KV launch.  Three
    query rows, so that both run the prefill kernel's key-chunk launch (with
    one or two rows the contiguous launch runs the decoding-shaped kernel)."""
    B, H, L, d, P = 2, 4, 1024, 128, 128
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((B, L, H, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    v = torch.from_numpy(rng.standard_normal((B, L, H, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    q = torch.from_numpy(rng.standard_normal((B, H, 3, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    kc = k.reshape(B * L // P, P, H, d)
    vc = v.reshape(B * L // P, P, H, d)
    table = torch.arange(B * L // P, dtype=torch.int32, device="cuda").reshape(B, L // P)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o1, l1 = gpu_lib.forward_paged(q, kc, vc, table, lens, num_splits=4)
    o2, l2 = gpu_lib.forward_splitkv(q, k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous(),
                                     num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(o1, o2)


# ---------------------------------------------------------------- 8-bit caches

QCASES = [
    # B, H, Nq, d, dtype, page_size, lens, splits, kind
    (3, 4, 1, 128, "bf16", 64, [1000, 70, 513], 4, "e4m3"),
    (2, 2, 5, 128, "f16", 128, [2048, 1], 3, "int8"),
    (4, 2, 1, 64, "bf16", 64, [300, 0, 64, 129], 3, "int8"),
    (2, 2, 2, 256, "bf16", 128, [900, 777], 2, "e4m3"),
    (2, 8, 1, 128, "bf16", 256, [8192, 3000], None, "e4m3"),
    (2, 2, 8, 64, "f16", 64, [1000, 65], 3, "e4m3"),
    (1, 4, 4, 256, "bf16", 128, [1500], 2, "int8"),
    (3, 2, 1, 256, "bf16", 64, [64, 0, 2500], 4, "e4m3"),
]


@pytest.mark.parametrize("B,H,Nq,d,dtype,page_size,lens,splits,kind", QCASES)
def test_paged_8bit_vs_oracle(gpu_lib, B, H, Nq, d, dtype, page_size, lens, splits, kind):
    import workloads as W

    seed = sum(lens) + d + len(kind)
    kc32, _, table = make_cache(B, H, lens, d, page_size, dtype, seed)  # only the table and cache shape
    n_pages, P = kc32.shape[0], kc32.shape[1]
    if kind == "e4m3":
        kcodes = W.random_e4m3_codes(kc32.shape, seed + 1)
        vcodes = W.random_e4m3_codes(kc32.shape, seed + 2)
        ks = W.random_scales(kc32.shape[:3], seed + 3, 0.02, 0.05)
        vs = W.random_scales(kc32.shape[:3], seed + 4, 0.02, 0.05)
    else:
        rng = np.random.default_rng(seed)
        kcodes = rng.integers(0, 256, size=kc32.shape, dtype=np.uint8)
        vcodes = rng.integers(0, 256, size=kc32.shape, dtype=np.uint8)
        ks = W.random_scales(kc32.shape[:3], seed + 3, 0.005, 0.01)
        vs = W.random_scales(kc32.shape[:3], seed + 4, 0.005, 0.01)
    rng = np.random.default_rng(seed + 5)
    qd, q = to_device(rng.standard_normal((B, H, Nq, d), dtype=np.float32), dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o, lse = gpu_lib.forward_paged(qd, t(kcodes), t(vcodes), t(table), torch.tensor(lens, dtype=torch.int32).cuda(),
                                   k_scale=t(ks), v_scale=t(vs), kv_dtype=kind, num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = PG.attention_paged_quant(q, kcodes, vcodes, ks, vs, table, np.array(lens), 1.0 / np.sqrt(d), kind)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, dtype,
          f"paged {kind} B{B} H{H} Nq{Nq} d{d} P{page_size} lens{lens} S{splits}")
    assert n_pages * P >= max(lens)


def test_paged_8bit_equals_16bit_cache(gpu_lib):
    """int8 codes with scale 1 are small integers: the same values stored as a
    bf16 cache give the same attention (both exact inputs to the kernel; the
    8-bit path only adds the multiplications by 1).  Three query rows: both
    caches on the prefill kernel's key-chunk launch."""
    B, H, d, P = 2, 4, 128, 128
    lens = [1000, 333]
    kc32, _, table = make_cache(B, H, lens, d, P, "bf16", 21)
    rng = np.random.default_rng(21)
    kcodes = rng.integers(-3, 4, size=kc32.shape).astype(np.int8)
    vcodes = rng.integers(-3, 4, size=kc32.shape).astype(np.int8)
    ones = torch.ones(kc32.shape[:3], dtype=torch.float32, device="cuda")
    q = torch.from_numpy(rng.standard_normal((B, H, 3, d), dtype=np.float32) * 0.1).to(torch.bfloat16).cuda()
    td = torch.from_numpy(table).cuda()
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    k8 = torch.from_numpy(kcodes.view(np.uint8)).cuda()
    v8 = torch.from_numpy(vcodes.view(np.uint8)).cuda()
    o1, l1 = gpu_lib.forward_paged(q, k8, v8, td, ld, k_scale=ones, v_scale=ones, kv_dtype="int8", num_splits=2)
    kb = torch.from_numpy(kcodes.astype(np.float32)).to(torch.bfloat16).cuda()
    vb = torch.from_numpy(vcodes.astype(np.float32)).to(torch.bfloat16).cuda()
    o2, l2 = gpu_lib.forward_paged(q, kb, vb, td, ld, num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(o1, o2)


@pytest.mark.parametrize("kind", ["int8", "e4m3"])
def test_decode_kernel_8bit_cache_equals_dense(gpu_lib, kind):
    """The decoding-shaped kernel (one query row) on an 8-bit paged cache with
    unit scales and pages in order equals the same kernel on the dense,
    contiguous copy of the decoded values: the codes widen to fp32 exactly,
    the scales multiply by 1, and both launches cut the keys at the same
    chunk bounds (1024 keys, 4 chunks)."""
    import workloads as W

    B, H, L, d, P = 2, 4, 1024, 128, 128
    rng = np.random.default_rng(5)
    if kind == "int8":
        kcodes = rng.integers(-100, 101, size=(B, L, H, d)).astype(np.int8).view(np.uint8)
        vcodes = rng.integers(-100, 101, size=(B, L, H, d)).astype(np.int8).view(np.uint8)
        dec = lambda c: c.view(np.int8).astype(np.float32)  # noqa: E731
    else:
        kcodes = W.random_e4m3_codes((B, L, H, d), 6)
        vcodes = W.random_e4m3_codes((B, L, H, d), 7)
        dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()  # noqa: E731
    q = torch.from_numpy(rng.standard_normal((B, H, 1, d), dtype=np.float32) * 0.02).to(torch.bfloat16).cuda()
    ones = torch.ones((B * L // P, P, H), dtype=torch.float32, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    table = torch.arange(B * L // P, dtype=torch.int32, device="cuda").reshape(B, L // P)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o1, l1 = gpu_lib.forward_paged(q, t(kcodes.reshape(B * L // P, P, H, d)), t(vcodes.reshape(B * L // P, P, H, d)),
                                   table, lens, k_scale=ones, v_scale=ones, kv_dtype=kind, num_splits=4)
    # the decoded values are exact in bfloat16 (e4m3 and small integers)
    kd = torch.from_numpy(dec(kcodes).transpose(0, 2, 1, 3).copy()).to(torch.bfloat16).cuda()
    vd = torch.from_numpy(dec(vcodes).transpose(0, 2, 1, 3).copy()).to(torch.bfloat16).cuda()
    o2, l2 = gpu_lib.forward_splitkv(q, kd, vd, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(o1, o2)


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
def test_paged_offsets_beyond_2_31(gpu_lib, kind):
    """A cache of more than 2^31 elements (40000 pages of 256 tokens, H2,
    d128: page p starts at element 65536 p, past 2^31 from page 32768) read
    through a table of 1025 pages drawn across the whole cache.  The
    sequence has 4099 * 64 keys (the last page holds 192); key g of head h
    is row g mod 4099 of that head's seeded bank (bf16 values, or e4m3 codes
    with per-(token, head) scales), so each (key, value) pair appears m = 64
    times: O equals attention over the bank alone and lse is ln m above its
    lse."""
    import workloads as W
    from oracle import exact as OX

    H, nq, d, P, n_pages, R, m = 2, 3, 128, 256, 40000, 4099, 64
    L = R * m
    n_used = -(-L // P)
    rng = np.random.default_rng(17)
    phys = rng.choice(n_pages, n_used, replace=False).astype(np.int64)
    assert phys.max() * P * H * d > 2 ** 31
    qd, q = to_device(rng.standard_normal((1, H, nq, d), dtype=np.float32), "bf16")
    gi = torch.arange(n_used * P, dtype=torch.int64, device="cuda") % R
    pt = torch.from_numpy(phys).cuda()

    def paged(bank_d, dtype):  # [H, R, ...] bank -> [n_pages, P, H, ...] cache with the sequence's pages at phys
        c = torch.zeros((n_pages, P, H) + tuple(bank_d.shape[2:]), dtype=dtype, device="cuda")
        src = bank_d.index_select(1, gi).view((H, n_used, P) + tuple(bank_d.shape[2:]))
        c[pt] = src.permute((1, 2, 0) + tuple(range(3, src.dim()))).contiguous()
        return c

    table = torch.from_numpy(phys.astype(np.int32)[None]).cuda()
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(d)
    if kind == "bf16":
        kb_d, kb = to_device(rng.standard_normal((H, R, d), dtype=np.float32), "bf16")
        vb_d, vb = to_device(rng.standard_normal((H, R, d), dtype=np.float32), "bf16")
        kc, vc = paged(kb_d, torch.bfloat16), paged(vb_d, torch.bfloat16)
        o, lse = gpu_lib.forward_paged(qd, kc, vc, table, lens, scale=scale)
    else:
        kcodes, vcodes = W.random_e4m3_codes((H, R, d), 21), W.random_e4m3_codes((H, R, d), 22)
        ks, vs = W.random_scales((H, R), 23, 0.02, 0.05), W.random_scales((H, R), 24, 0.02, 0.05)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        kc, vc = paged(t(kcodes), torch.uint8), paged(t(vcodes), torch.uint8)
        ksc, vsc = paged(t(ks), torch.float32), paged(t(vs), torch.float32)
        o, lse = gpu_lib.forward_paged(qd, kc, vc, table, lens, scale=scale, k_scale=ksc, v_scale=vsc,
                                       kv_dtype="e4m3")
        kb, vb = PG.dequantize(kcodes, ks, "e4m3"), PG.dequantize(vcodes, vs, "e4m3")
        del ksc, vsc
    torch.cuda.synchronize()
    o_n, lse_n = o.double().cpu().numpy(), lse.double().cpu().numpy()
    del kc, vc, o, lse
    torch.cuda.empty_cache()
    for h in range(H):
        o_ref, l_ref = OX.attention_rows(q[0, h], kb[h], vb[h], np.arange(nq), scale, False)
        check(o_n[0, h], lse_n[0, h], o_ref, l_ref + np.log(m), "bf16", f"paged {kind} offsets beyond 2^31, head {h}")


# ---------------------------------------------------------------- e4m3 queries

FP8Q_CASES = [
    # B, H, Nq, d, page_size, lens, splits, kind
    (3, 4, 1, 128, 64, [1000, 70, 513], 4, "e4m3"),
    (2, 2, 2, 128, 128, [2048, 1], 3, "int8"),
    (4, 2, 1, 64, 64, [300, 0, 64, 129], 3, "e4m3"),
    (2, 2, 2, 256, 128, [900, 777], 2, "e4m3"),
    (1, 4, 1, 256, 64, [1500], 5, "int8"),
    (2, 8, 1, 128, 256, [8192, 3000], None, "e4m3"),
]


def _fp8_query(B, H, Nq, d, seed):
    """e4m3 query codes and one scale per (batch, head), and the query values
    they stand for (decoded by the oracle, in fp64)."""
    import workloads as W
    from oracle.fp8 import e4m3_decode

    codes = W.random_e4m3_codes((B, H, Nq, d), seed)
    qs = W.random_scales((B, H), seed + 1, 0.5, 2.0)
    return codes, qs, e4m3_decode(codes) * qs.astype(np.float64)[:, :, None, None]


@pytest.mark.parametrize("B,H,Nq,d,page_size,lens,splits,kind", FP8Q_CASES)
def test_paged_fp8_queries_vs_oracle(gpu_lib, B, H, Nq, d, page_size, lens, splits, kind):
    """attn_fwd_paged_fp8: e4m3 queries (one scale per batch and head) on the
    decoding-shaped kernel over an 8-bit cache, against the oracle's paged
    attention on the decoded queries; output bf16."""
    import workloads as W

    seed = sum(lens) + d + 3 * Nq
    kc32, _, table = make_cache(B, H, lens, d, page_size, "bf16", seed)
    if kind == "e4m3":
        kcodes = W.random_e4m3_codes(kc32.shape, seed + 1)
        vcodes = W.random_e4m3_codes(kc32.shape, seed + 2)
        ks = W.random_scales(kc32.shape[:3], seed + 3, 0.02, 0.05)
        vs = W.random_scales(kc32.shape[:3], seed + 4, 0.02, 0.05)
    else:
        rng = np.random.default_rng(seed)
        kcodes = rng.integers(0, 256, size=kc32.shape, dtype=np.uint8)
        vcodes = rng.integers(0, 256, size=kc32.shape, dtype=np.uint8)
        ks = W.random_scales(kc32.shape[:3], seed + 3, 0.005, 0.01)
        vs = W.random_scales(kc32.shape[:3], seed + 4, 0.005, 0.01)
    qcodes, qs, q64 = _fp8_query(B, H, Nq, d, seed + 5)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o, lse = gpu_lib.forward_paged_fp8(t(qcodes), t(qs), t(kcodes), t(vcodes), t(table),
                                       torch.tensor(lens, dtype=torch.int32).cuda(), k_scale=t(ks), v_scale=t(vs),
                                       kv_dtype=kind, num_splits=splits)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ref_o, ref_l = PG.attention_paged_quant(q64, kcodes, vcodes, ks, vs, table, np.array(lens), 1.0 / np.sqrt(d), kind)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, "bf16",
          f"paged fp8 queries {kind} B{B} H{H} Nq{Nq} d{d} P{page_size} lens{lens} S{splits}")


@pytest.mark.parametrize("nq", [1, 2])
def test_paged_fp8_queries_unit_scale_equal_bf16_queries(gpu_lib, nq):
    """e4m3 query codes with scale 1 and the same values as bf16 queries (e4m3
    values are exact in bf16) give bitwise the same result: both run the
    decoding-shaped kernel, whose query is value * c in fp32 either way."""
    import workloads as W

    B, H, d, P = 2, 4, 128, 128
    lens = [1500, 333]
    kc32, _, table = make_cache(B, H, lens, d, P, "bf16", 31)
    kcodes = W.random_e4m3_codes(kc32.shape, 32)
    vcodes = W.random_e4m3_codes(kc32.shape, 33)
    ks = W.random_scales(kc32.shape[:3], 34, 0.02, 0.05)
    vs = W.random_scales(kc32.shape[:3], 35, 0.02, 0.05)
    qcodes = W.random_e4m3_codes((B, H, nq, d), 36)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    td, ld = t(table), torch.tensor(lens, dtype=torch.int32).cuda()
    o1, l1 = gpu_lib.forward_paged_fp8(t(qcodes), torch.ones((B, H), dtype=torch.float32, device="cuda"), t(kcodes),
                                       t(vcodes), td, ld, k_scale=t(ks), v_scale=t(vs), kv_dtype="e4m3", num_splits=3)
    qb = t(qcodes).view(torch.float8_e4m3fn).to(torch.bfloat16)
    o2, l2 = gpu_lib.forward_paged(qb, t(kcodes), t(vcodes), td, ld, k_scale=t(ks), v_scale=t(vs), kv_dtype="e4m3",
                                   num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(o1, o2)


def test_paged_fp8_queries_full_decode_shape(gpu_lib):
    """The benchmark's decoding shape with e4m3 queries over an e4m3 cache (B2
    H32 d128, 256-token pages in shuffled order, default chunk count), one
    sequence at the full 32768 tokens and one ragged; four of the 32 heads
    checked against the oracle (heads are independent, so the oracle reads
    only their slice of the cache)."""
    import workloads as W

    B, H, d, P = 2, 32, 128, 256
    lens = [32768, 20001]
    kc32, _, table = make_cache(B, 1, lens, d, P, "bf16", 41, spare=3)  # table and page count only
    shape = (kc32.shape[0], P, H, d)
    kcodes, vcodes = W.random_e4m3_codes(shape, 42), W.random_e4m3_codes(shape, 43)
    ks, vs = W.random_scales(shape[:3], 44, 0.02, 0.05), W.random_scales(shape[:3], 45, 0.02, 0.05)
    qcodes, qs, q64 = _fp8_query(B, H, 1, d, 46)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o, lse = gpu_lib.forward_paged_fp8(t(qcodes), t(qs), t(kcodes), t(vcodes), t(table),
                                       torch.tensor(lens, dtype=torch.int32).cuda(), k_scale=t(ks), v_scale=t(vs),
                                       kv_dtype="e4m3")
    torch.cuda.synchronize()
    heads = [0, 7, 20, 31]
    ref_o, ref_l = PG.attention_paged_quant(q64[:, heads], kcodes[:, :, heads], vcodes[:, :, heads],
                                            ks[:, :, heads], vs[:, :, heads], table, np.array(lens),
                                            1.0 / np.sqrt(d), "e4m3")
    check(o[:, heads].double().cpu().numpy(), lse[:, heads].double().cpu().numpy(), ref_o, ref_l, "bf16",
          "paged fp8 queries, decoding shape B2 H32 Nk32768")
