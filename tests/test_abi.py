"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before touching the device (CPU only).

No call here reaches a kernel launch: every argument set is invalid, and
validation returns before any HIP call, so these run without a GPU.
"""

import ctypes
import os
import re

import pytest

import exact_attention_forward_03_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # a non-null, 64 KiB-aligned address; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.lib_path()):
        pytest.fail("libattn.so is not built (run __graft_entry__.build())")
    return attn.load()


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(attn.EXPORTS)


def test_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(attn.lib_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_strerror(lib):
    assert attn.attn_strerror(attn.ATTN_OK) == "ATTN_OK"
    for code in (attn.ATTN_ERR_INVALID_ARG, attn.ATTN_ERR_UNSUPPORTED, attn.ATTN_ERR_HIP, attn.ATTN_ERR_TOO_LARGE):
        assert "ATTN_ERR" in attn.attn_strerror(code)
    assert "unknown" in attn.attn_strerror(12345)


def good_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Nq=256, Nk=256, d=64, scale=0.125,
             causal=0, cu_seqlens_q=None, cu_seqlens_k=None, dtype=attn.ATTN_DT_F16,
             q_scale=None, k_scale=None, v_scale=None)
    a.update(over)
    return a


def call_fwd(**over):
    a = good_args(**over)
    return attn.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                         a["scale"], a["causal"], a["cu_seqlens_q"], a["cu_seqlens_k"], a["dtype"],
                         a["q_scale"], a["k_scale"], a["v_scale"])


def call_fwd_stream(**over):
    a = good_args(**over)
    return attn.attn_fwd_stream(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                                a["d"], a["scale"], a["causal"], a["cu_seqlens_q"], a["cu_seqlens_k"],
                                a["dtype"], a["q_scale"], a["k_scale"], a["v_scale"], None)


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(k=None, v=None, Nq=0), dict(q=None, Nk=0),
    dict(B=0), dict(H=0), dict(B=-1), dict(Nq=-1), dict(Nk=-5),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=-0.5),
    dict(causal=2), dict(causal=-1),
    dict(cu_seqlens_q=FAKE), dict(cu_seqlens_k=FAKE),
    dict(dtype=7), dict(dtype=-1), dict(dtype=attn.ATTN_DT_F32),
    dict(dtype=attn.ATTN_DT_FP8_E4M3, d=128),  # fp8 without scales
    dict(dtype=attn.ATTN_DT_FP8_E4M3, d=128, q_scale=FAKE, k_scale=FAKE),
    dict(q=FAKE + 8), dict(o=FAKE + 2), dict(lse=FAKE + 2),
    dict(cu_seqlens_q=FAKE + 2, cu_seqlens_k=FAKE),
]


@pytest.mark.parametrize("over", INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
@pytest.mark.parametrize("entry", [call_fwd, call_fwd_stream], ids=["attn_fwd", "attn_fwd_stream"])
def test_invalid_arguments(lib, entry, over):
    assert entry(**over) == attn.ATTN_ERR_INVALID_ARG


UNSUPPORTED = [
    dict(d=96), dict(d=32), dict(d=512), dict(d=0),
    dict(dtype=attn.ATTN_DT_FP8_E4M3, d=96, q_scale=FAKE, k_scale=FAKE, v_scale=FAKE),
    dict(dtype=attn.ATTN_DT_FP8_E4M3, d=512, q_scale=FAKE, k_scale=FAKE, v_scale=FAKE,
         cu_seqlens_q=FAKE, cu_seqlens_k=FAKE),
]


@pytest.mark.parametrize("over", UNSUPPORTED, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_unsupported(lib, over):
    assert call_fwd(**over) == attn.ATTN_ERR_UNSUPPORTED


def test_empty_query_is_a_noop(lib):
    # Nq = 0 returns before any HIP call
    assert call_fwd(Nq=0) == attn.ATTN_OK
    assert call_fwd(Nq=0, Nk=0) == attn.ATTN_OK
    assert call_fwd(Nq=0, q=None, o=None, lse=None) == attn.ATTN_OK


def quant(**over):
    a = dict(x=FAKE, x_dtype=attn.ATTN_DT_F32, x_fp8=FAKE, x_scale=FAKE, B=1, H=1, N=128, d=128,
             signs=None, per_tensor=0)
    a.update(over)
    return attn.attn_fp8_quantize(a["x"], a["x_dtype"], a["x_fp8"], a["x_scale"], a["B"], a["H"], a["N"],
                                  a["d"], a["signs"], a["per_tensor"], None)


@pytest.mark.parametrize("over", [dict(x=None), dict(x_fp8=None), dict(x_scale=None), dict(B=0), dict(H=0),
                                  dict(N=-1), dict(x_dtype=attn.ATTN_DT_FP8_E4M3), dict(x_dtype=9),
                                  dict(per_tensor=2), dict(x=FAKE + 4), dict(x_scale=FAKE + 1),
                                  dict(signs=FAKE + 2)],
                         ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_quantize_invalid(lib, over):
    assert quant(**over) == attn.ATTN_ERR_INVALID_ARG


def test_quantize_unsupported_and_noop(lib):
    assert quant(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert quant(N=0) == attn.ATTN_OK


def quant_varlen(**over):
    a = dict(x=FAKE, x_dtype=attn.ATTN_DT_F32, x_fp8=FAKE, x_scale=FAKE, H=2, T=300, d=128, cu=FAKE, nseq=3,
             signs=None, per_tensor=0)
    a.update(over)
    return attn.attn_fp8_quantize_varlen(a["x"], a["x_dtype"], a["x_fp8"], a["x_scale"], a["H"], a["T"], a["d"],
                                         a["cu"], a["nseq"], a["signs"], a["per_tensor"], None)


@pytest.mark.parametrize("over", [dict(x=None), dict(x_fp8=None), dict(x_scale=None), dict(cu=None), dict(H=0),
                                  dict(T=-1), dict(nseq=0), dict(x_dtype=attn.ATTN_DT_FP8_E4M3),
                                  dict(per_tensor=2), dict(x=FAKE + 4), dict(cu=FAKE + 2), dict(signs=FAKE + 2),
                                  dict(T=2 ** 31 - 1, nseq=2 ** 30, H=4)],
                         ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_quantize_varlen_invalid(lib, over):
    assert quant_varlen(**over) == attn.ATTN_ERR_INVALID_ARG


def test_quantize_varlen_unsupported_and_noop(lib):
    assert quant_varlen(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert quant_varlen(T=0) == attn.ATTN_OK


def test_binding_has_no_cpu_fallback():
    """The torch front end goes through the library only: no oracle import."""
    src = open(os.path.join(ROOT, "exact_attention_forward_03_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no oracle", "")
    for f in os.listdir(os.path.join(ROOT, "exact_attention_forward_03_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "exact_attention_forward_03_amd", "csrc", f)).read()


def split_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Nq=1, Nk=4096, d=128, scale=0.125, causal=0,
             dtype=attn.ATTN_DT_BF16, num_splits=8, o_part=FAKE, lse_part=FAKE)
    a.update(over)
    return attn.attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                                 a["d"], a["scale"], a["causal"], a["dtype"], a["num_splits"], a["o_part"],
                                 a["lse_part"], None)


SPLIT_INVALID = [
    dict(q=None), dict(o=None), dict(lse=None), dict(k=None), dict(B=0), dict(Nq=-1), dict(Nk=-1),
    dict(scale=float("nan")), dict(causal=3), dict(dtype=5), dict(num_splits=0), dict(num_splits=-2),
    dict(num_splits=1025), dict(o_part=None), dict(lse_part=None), dict(o_part=FAKE + 4),
    dict(lse_part=FAKE + 2), dict(q=FAKE + 8),
]


@pytest.mark.parametrize("over", SPLIT_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_splitkv_invalid(lib, over):
    assert split_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_splitkv_unsupported_and_empty(lib):
    assert split_call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert split_call(dtype=attn.ATTN_DT_FP8_E4M3) == attn.ATTN_ERR_UNSUPPORTED
    assert split_call(Nq=0) == attn.ATTN_OK
    assert split_call(Nq=0, q=None, o=None, lse=None, o_part=None, lse_part=None) == attn.ATTN_OK


def split8_call(**over):
    a = dict(q8=FAKE, q_scale=FAKE, k8=FAKE, k_scale=FAKE, v8=FAKE, v_scale=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Nq=256,
             Nk=4096, d=128, scale=0.125, causal=0, num_splits=8, o_part=FAKE, lse_part=FAKE)
    a.update(over)
    return attn.attn_fwd_splitkv_fp8(a["q8"], a["q_scale"], a["k8"], a["k_scale"], a["v8"], a["v_scale"], a["o"],
                                     a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                     a["num_splits"], a["o_part"], a["lse_part"], None)


SPLIT8_INVALID = [
    dict(q8=None), dict(o=None), dict(lse=None), dict(k8=None), dict(v8=None), dict(q_scale=None),
    dict(k_scale=None), dict(v_scale=None), dict(B=0), dict(Nq=-1), dict(Nk=-1), dict(scale=float("nan")),
    dict(scale=-1.0), dict(causal=2), dict(num_splits=0), dict(num_splits=1025), dict(o_part=None),
    dict(lse_part=None), dict(o_part=FAKE + 4), dict(lse_part=FAKE + 2), dict(q8=FAKE + 8), dict(k_scale=FAKE + 2),
]


@pytest.mark.parametrize("over", SPLIT8_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_splitkv_fp8_invalid(lib, over):
    assert split8_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_splitkv_fp8_unsupported_and_empty(lib):
    assert split8_call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert split8_call(Nq=0) == attn.ATTN_OK
    assert split8_call(Nq=0, q8=None, q_scale=None, o=None, lse=None, o_part=None, lse_part=None) == attn.ATTN_OK


def noalloc_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Nq=1, Nk=4096, d=128, scale=0.125, causal=0,
             dtype=attn.ATTN_DT_BF16, num_splits=8)
    a.update(over)
    return attn.attn_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                         a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["num_splits"], None)


NOALLOC_INVALID = [o for o in SPLIT_INVALID if "o_part" not in o and "lse_part" not in o]


@pytest.mark.parametrize("over", NOALLOC_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_splitkv_noalloc_invalid(lib, over):
    assert noalloc_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_splitkv_noalloc_limits(lib):
    """The fixed scratch holds num_splits * B * H * Nq rows of d + 1 fp32
    values (O parts rounded up to 256 bytes): calls past it return
    ATTN_ERR_TOO_LARGE before any HIP call (none of these reaches the
    device), as do sizes whose product would overflow."""
    cap = attn.ATTN_NOALLOC_SCRATCH_BYTES
    assert cap == 32 << 20
    rows_max = cap // (129 * 4)  # d = 128, ignoring the 256-byte rounding
    assert noalloc_call(B=1, H=1, Nq=rows_max + 1, num_splits=1) == attn.ATTN_ERR_TOO_LARGE
    assert noalloc_call(B=64, H=64, Nq=64, num_splits=8) == attn.ATTN_ERR_TOO_LARGE
    assert noalloc_call(B=2 ** 20, H=2 ** 9, Nq=2 ** 30, num_splits=1024) == attn.ATTN_ERR_TOO_LARGE
    assert noalloc_call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert noalloc_call(dtype=attn.ATTN_DT_FP8_E4M3) == attn.ATTN_ERR_UNSUPPORTED
    assert noalloc_call(Nq=0) == attn.ATTN_OK
    assert noalloc_call(Nq=0, q=None, o=None, lse=None) == attn.ATTN_OK
    assert "scratch" in attn.attn_strerror(attn.ATTN_ERR_TOO_LARGE)


def merge_call(**over):
    a = dict(o_part=FAKE, lse_part=FAKE, num_splits=4, B=1, H=2, Nq=16, d=128, o=FAKE, lse=FAKE,
             o_dtype=attn.ATTN_DT_BF16)
    a.update(over)
    return attn.attn_merge(a["o_part"], a["lse_part"], a["num_splits"], a["B"], a["H"], a["Nq"], a["d"], a["o"],
                           a["lse"], a["o_dtype"], None)


MERGE_INVALID = [
    dict(o_part=None), dict(lse_part=None), dict(o=None), dict(lse=None), dict(num_splits=0),
    dict(num_splits=2000), dict(B=0), dict(H=-1), dict(Nq=-3), dict(o_dtype=attn.ATTN_DT_F32),
    dict(o_dtype=attn.ATTN_DT_FP8_E4M3), dict(o_part=FAKE + 8), dict(o=FAKE + 2), dict(lse=FAKE + 1),
]


@pytest.mark.parametrize("over", MERGE_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_merge_invalid(lib, over):
    assert merge_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_merge_unsupported_and_empty(lib):
    assert merge_call(d=80) == attn.ATTN_ERR_UNSUPPORTED
    assert merge_call(Nq=0) == attn.ATTN_OK
    assert merge_call(Nq=0, o_part=None, lse_part=None, o=None, lse=None) == attn.ATTN_OK


def bwd_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE, B=1, H=2,
             Nq=256, Nk=256, d=128, scale=0.125, causal=0, cu_q=None, cu_k=None, dtype=attn.ATTN_DT_BF16)
    a.update(over)
    return attn.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["delta"],
                         a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["cu_q"], a["cu_k"],
                         a["dtype"], None)


BWD_INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None), dict(dout=None), dict(dq=None),
    dict(dk=None), dict(dv=None), dict(delta=None), dict(B=0), dict(H=0), dict(Nq=-1), dict(Nk=-5),
    dict(scale=float("inf")), dict(scale=-1.0), dict(causal=2), dict(dtype=7), dict(q=FAKE + 8),
    dict(dout=FAKE + 4), dict(dq=FAKE + 2), dict(dk=FAKE + 8), dict(dv=FAKE + 8), dict(o=FAKE + 8),
    dict(lse=FAKE + 2), dict(delta=FAKE + 1), dict(cu_q=FAKE), dict(cu_k=FAKE), dict(cu_q=FAKE + 2, cu_k=FAKE),
]


@pytest.mark.parametrize("over", BWD_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_bwd_invalid(lib, over):
    assert bwd_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_bwd_unsupported_and_empty(lib):
    assert bwd_call(d=80) == attn.ATTN_ERR_UNSUPPORTED
    assert bwd_call(dtype=attn.ATTN_DT_FP8_E4M3) == attn.ATTN_ERR_UNSUPPORTED
    # no queries and no keys: nothing to write, no launch
    none = dict(q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None, dv=None, delta=None)
    assert bwd_call(Nq=0, Nk=0, **none) == attn.ATTN_OK


def bwd8_call(**over):
    a = dict(q8=FAKE, sq=FAKE, k8=FAKE, sk=FAKE, v8=FAKE, sv=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE,
             dv=FAKE, stats=FAKE, do8=FAKE, sdo=FAKE, B=1, H=2, Nq=256, Nk=256, d=128, scale=0.125, causal=0)
    a.update(over)
    return attn.attn_bwd_fp8(a["q8"], a["sq"], a["k8"], a["sk"], a["v8"], a["sv"], a["o"], a["lse"], a["dout"],
                             a["dq"], a["dk"], a["dv"], a["stats"], a["do8"], a["sdo"], a["B"], a["H"], a["Nq"],
                             a["Nk"], a["d"], a["scale"], a["causal"], None)


BWD8_INVALID = [dict(**{k: None}) for k in ("q8", "sq", "k8", "sk", "v8", "sv", "o", "lse", "dout", "dq", "dk", "dv",
                                            "stats", "do8", "sdo")] + [
    dict(B=0), dict(H=0), dict(Nq=-1), dict(Nk=-1), dict(scale=float("nan")), dict(scale=-0.5), dict(causal=3),
    dict(q8=FAKE + 8), dict(k8=FAKE + 4), dict(v8=FAKE + 1), dict(o=FAKE + 8), dict(dout=FAKE + 2),
    dict(dq=FAKE + 8), dict(dk=FAKE + 8), dict(dv=FAKE + 8), dict(do8=FAKE + 8), dict(sq=FAKE + 2),
    dict(sk=FAKE + 1), dict(sv=FAKE + 3), dict(lse=FAKE + 2), dict(stats=FAKE + 2), dict(sdo=FAKE + 1),
    dict(B=1 << 16, H=1 << 14, Nq=1 << 12),  # more than 2^31 - 1 workgroups
]


@pytest.mark.parametrize("over", BWD8_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_bwd_fp8_invalid(lib, over):
    assert bwd8_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_bwd_fp8_unsupported_and_empty(lib):
    for d in (64, 256, 80):
        assert bwd8_call(d=d) == attn.ATTN_ERR_UNSUPPORTED
    none = {k: None for k in ("q8", "sq", "k8", "sk", "v8", "sv", "o", "lse", "dout", "dq", "dk", "dv", "stats",
                              "do8", "sdo")}
    assert bwd8_call(Nq=0, Nk=0, **none) == attn.ATTN_OK


def paged_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, table=FAKE, lens=FAKE, o=FAKE, lse=FAKE, B=2, H=4, Nq=1, d=128,
             num_pages=64, page_size=128, max_pages=16, scale=0.125, dtype=attn.ATTN_DT_BF16, kv_dtype=None,
             num_splits=4, o_part=FAKE, lse_part=FAKE)
    a.update(over)
    kvd = a["dtype"] if a["kv_dtype"] is None else a["kv_dtype"]
    return attn.attn_fwd_paged(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["table"], a["lens"], a["o"], a["lse"],
                               a["B"], a["H"], a["Nq"], a["d"], a["num_pages"], a["page_size"], a["max_pages"],
                               a["scale"], a["dtype"], kvd, a["num_splits"], a["o_part"], a["lse_part"], None)


PAGED_INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(table=None), dict(lens=None), dict(o=None), dict(lse=None),
    dict(o_part=None), dict(lse_part=None), dict(B=0), dict(H=0), dict(Nq=-1), dict(num_pages=0),
    dict(page_size=0), dict(max_pages=0), dict(scale=float("nan")), dict(dtype=9), dict(num_splits=0),
    dict(num_splits=1025), dict(q=FAKE + 8), dict(k=FAKE + 8), dict(table=FAKE + 2), dict(lens=FAKE + 1),
    dict(o_part=FAKE + 4), dict(max_pages=1 << 24, page_size=1 << 10),
    dict(kv_dtype=attn.ATTN_DT_F16), dict(kv_dtype=attn.ATTN_DT_F32),
    dict(kv_dtype=attn.ATTN_DT_INT8), dict(kv_dtype=attn.ATTN_DT_FP8_E4M3, ks=FAKE),
    dict(kv_dtype=attn.ATTN_DT_INT8, ks=FAKE, vs=FAKE + 2),
]


@pytest.mark.parametrize("over", PAGED_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_paged_invalid(lib, over):
    assert paged_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_paged_unsupported_and_empty(lib):
    assert paged_call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert paged_call(page_size=96) == attn.ATTN_ERR_UNSUPPORTED
    assert paged_call(page_size=16) == attn.ATTN_ERR_UNSUPPORTED
    assert paged_call(dtype=attn.ATTN_DT_FP8_E4M3, ks=FAKE, vs=FAKE) == attn.ATTN_ERR_UNSUPPORTED
    assert paged_call(Nq=0) == attn.ATTN_OK
    none = dict(q=None, k=None, v=None, table=None, lens=None, o=None, lse=None, o_part=None, lse_part=None)
    assert paged_call(Nq=0, **none) == attn.ATTN_OK


def paged8_call(**over):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, table=FAKE, lens=FAKE, o=FAKE, lse=FAKE, B=2, H=4,
             Nq=1, d=128, num_pages=64, page_size=128, max_pages=16, scale=0.125, kv_dtype=attn.ATTN_DT_FP8_E4M3,
             num_splits=4, o_part=FAKE, lse_part=FAKE)
    a.update(over)
    return attn.attn_fwd_paged_fp8(a["q"], a["qs"], a["k"], a["v"], a["ks"], a["vs"], a["table"], a["lens"], a["o"],
                                   a["lse"], a["B"], a["H"], a["Nq"], a["d"], a["num_pages"], a["page_size"],
                                   a["max_pages"], a["scale"], a["kv_dtype"], a["num_splits"], a["o_part"],
                                   a["lse_part"], None)


PAGED8_INVALID = [
    dict(q=None), dict(qs=None), dict(k=None), dict(ks=None), dict(vs=None), dict(table=None), dict(o=None),
    dict(o_part=None), dict(B=0), dict(Nq=-1), dict(scale=-1.0), dict(num_splits=0), dict(qs=FAKE + 2),
    dict(q=FAKE + 8), dict(kv_dtype=attn.ATTN_DT_BF16), dict(kv_dtype=attn.ATTN_DT_F16), dict(kv_dtype=9),
]


@pytest.mark.parametrize("over", PAGED8_INVALID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_paged_fp8_invalid(lib, over):
    assert paged8_call(**over) == attn.ATTN_ERR_INVALID_ARG


def test_paged_fp8_unsupported_and_empty(lib):
    assert paged8_call(Nq=3) == attn.ATTN_ERR_UNSUPPORTED  # more rows than the decoding-shaped kernel takes
    assert paged8_call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert paged8_call(page_size=96) == attn.ATTN_ERR_UNSUPPORTED
    assert paged8_call(Nq=0) == attn.ATTN_OK
    none = dict(q=None, qs=None, k=None, v=None, ks=None, vs=None, table=None, lens=None, o=None, lse=None,
                o_part=None, lse_part=None)
    assert paged8_call(Nq=0, **none) == attn.ATTN_OK
