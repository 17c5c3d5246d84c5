"""Python binding of ``libattn.so`` (include/attn.h): exact attention forward
(and its gradients) on MI355X (gfx950).

The C entry points are exposed under their own names with plain integer
pointers (argument marshalling only): ``attn_fwd``, ``attn_fwd_stream``,
``attn_fwd_splitkv``, ``attn_fwd_splitkv_fp8``, ``attn_fwd_paged``, ``attn_fwd_paged_fp8``, ``attn_merge``,
``attn_bwd``,
``attn_bwd_fp8``, ``attn_fp8_quantize``, ``attn_fp8_quantize_varlen``,
``attn_strerror``.  ``forward``, ``forward_splitkv``, ``forward_splitkv_fp8``, ``forward_paged``,
``forward_paged_fp8``,
``merge``, ``backward``, ``backward_fp8``, ``fp8_quantize`` and
``fp8_quantize_varlen`` are the
torch-facing conveniences: they allocate the
outputs (and workspaces) with torch on the inputs' device, pass
``data_ptr()``s and torch's current HIP stream, and raise ``RuntimeError`` on
a non-zero return code.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = [
    "ATTN_DT_F16", "ATTN_DT_BF16", "ATTN_DT_FP8_E4M3", "ATTN_DT_F32", "ATTN_DT_INT8",
    "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_HIP", "ATTN_ERR_TOO_LARGE",
    "ATTN_NOALLOC_SCRATCH_BYTES", "attn_fwd_splitkv_noalloc", "forward_splitkv_noalloc",
    "load", "lib_path", "attn_fwd", "attn_fwd_stream", "attn_fwd_splitkv", "attn_merge", "attn_fp8_quantize",
    "attn_fwd_paged", "attn_bwd", "attn_bwd_fp8", "attn_strerror", "attn_fp8_quantize_varlen", "forward",
    "forward_splitkv", "forward_paged", "merge", "backward", "backward_fp8", "fp8_quantize", "fp8_quantize_varlen",
    "default_splits", "EXPORTS", "attn_fwd_splitkv_fp8", "forward_splitkv_fp8", "attn_fwd_paged_fp8",
    "forward_paged_fp8",
]

ATTN_DT_F16, ATTN_DT_BF16, ATTN_DT_FP8_E4M3, ATTN_DT_F32, ATTN_DT_INT8 = 0, 1, 2, 3, 4
ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP, ATTN_ERR_TOO_LARGE = 0, -1, -2, -3, -4
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20  # the fixed device scratch of attn_fwd_splitkv_noalloc (include/attn.h)

EXPORTS = ("attn_fwd", "attn_fwd_stream", "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc", "attn_fwd_splitkv_fp8",
           "attn_fwd_paged", "attn_fwd_paged_fp8",
           "attn_merge", "attn_bwd", "attn_bwd_fp8", "attn_fp8_quantize", "attn_fp8_quantize_varlen", "attn_strerror")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_FWD_ARGS = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _p, _i, _p, _p, _p]


def lib_path() -> str:
    return os.path.join(_HERE, "libattn.so")


def load():
    """Load libattn.so (built by ``__graft_entry__.build()``); raises if absent."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.attn_fwd.argtypes = _FWD_ARGS
        lib.attn_fwd.restype = _i
        lib.attn_fwd_stream.argtypes = _FWD_ARGS + [_p]
        lib.attn_fwd_stream.restype = _i
        lib.attn_fwd_splitkv.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p, _p, _p]
        lib.attn_fwd_splitkv.restype = _i
        lib.attn_fwd_splitkv_fp8.argtypes = [_p] * 8 + [_i] * 5 + [_f, _i, _i, _p, _p, _p]
        lib.attn_fwd_splitkv_fp8.restype = _i
        lib.attn_fwd_splitkv_noalloc.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _i, _i, _p]
        lib.attn_fwd_splitkv_noalloc.restype = _i
        lib.attn_merge.argtypes = [_p, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p]
        lib.attn_merge.restype = _i
        lib.attn_fwd_paged.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                                        _i, _p, _p, _p]
        lib.attn_fwd_paged.restype = _i
        lib.attn_fwd_paged_fp8.argtypes = [_p] * 10 + [_i] * 7 + [_f, _i, _i, _p, _p, _p]
        lib.attn_fwd_paged_fp8.restype = _i
        lib.attn_bwd.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _p, _i, _p]
        lib.attn_bwd.restype = _i
        lib.attn_bwd_fp8.argtypes = [_p] * 15 + [_i, _i, _i, _i, _i, _f, _i, _p]
        lib.attn_bwd_fp8.restype = _i
        lib.attn_fp8_quantize.argtypes = [_p, _i, _p, _p, _i, _i, _i, _i, _p, _i, _p]
        lib.attn_fp8_quantize.restype = _i
        lib.attn_fp8_quantize_varlen.argtypes = [_p, _i, _p, _p, _i, _i, _i, _p, _i, _p, _i, _p]
        lib.attn_fp8_quantize_varlen.restype = _i
        lib.attn_strerror.argtypes = [_i]
        lib.attn_strerror.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


# ---------------------------------------------------------------- C names

def attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q, cu_seqlens_k, dtype,
             q_scale, k_scale, v_scale) -> int:
    return load().attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q, cu_seqlens_k,
                           dtype, q_scale, k_scale, v_scale)


def attn_fwd_stream(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q, cu_seqlens_k, dtype,
                    q_scale, k_scale, v_scale, hip_stream) -> int:
    return load().attn_fwd_stream(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q,
                                  cu_seqlens_k, dtype, q_scale, k_scale, v_scale, hip_stream)


def attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits, o_part, lse_part,
                     hip_stream) -> int:
    return load().attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits, o_part,
                                   lse_part, hip_stream)


def attn_fwd_splitkv_fp8(q8, q_scale, k8, k_scale, v8, v_scale, o, lse, B, H, Nq, Nk, d, scale, causal,
                         num_splits, o_part, lse_part, hip_stream) -> int:
    return load().attn_fwd_splitkv_fp8(q8, q_scale, k8, k_scale, v8, v_scale, o, lse, B, H, Nq, Nk, d, scale,
                                       causal, num_splits, o_part, lse_part, hip_stream)


def attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits,
                             hip_stream) -> int:
    return load().attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits,
                                           hip_stream)


def attn_merge(o_part, lse_part, num_splits, B, H, Nq, d, o, lse, o_dtype, hip_stream) -> int:
    return load().attn_merge(o_part, lse_part, num_splits, B, H, Nq, d, o, lse, o_dtype, hip_stream)


def attn_fwd_paged(q, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k, o, lse, B, H, Nq, d, num_pages,
                   page_size, max_pages, scale, dtype, kv_dtype, num_splits, o_part, lse_part, hip_stream) -> int:
    return load().attn_fwd_paged(q, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k, o, lse, B, H, Nq, d,
                                 num_pages, page_size, max_pages, scale, dtype, kv_dtype, num_splits, o_part,
                                 lse_part, hip_stream)


def attn_fwd_paged_fp8(q8, q_scale, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k, o, lse, B, H, Nq, d,
                       num_pages, page_size, max_pages, scale, kv_dtype, num_splits, o_part, lse_part,
                       hip_stream) -> int:
    return load().attn_fwd_paged_fp8(q8, q_scale, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k, o, lse,
                                     B, H, Nq, d, num_pages, page_size, max_pages, scale, kv_dtype, num_splits, o_part,
                                     lse_part, hip_stream)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q, cu_seqlens_k,
             dtype, hip_stream) -> int:
    return load().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q,
                           cu_seqlens_k, dtype, hip_stream)


def attn_bwd_fp8(q8, q_scale, k8, k_scale, v8, v_scale, o, lse, dout, dq, dk, dv, stats, do8, do_scale, B, H, Nq,
                 Nk, d, scale, causal, hip_stream) -> int:
    return load().attn_bwd_fp8(q8, q_scale, k8, k_scale, v8, v_scale, o, lse, dout, dq, dk, dv, stats, do8,
                               do_scale, B, H, Nq, Nk, d, scale, causal, hip_stream)


def attn_fp8_quantize(x, x_dtype, x_fp8, x_scale, B, H, N, d, signs, per_tensor, hip_stream) -> int:
    return load().attn_fp8_quantize(x, x_dtype, x_fp8, x_scale, B, H, N, d, signs, per_tensor, hip_stream)


def attn_fp8_quantize_varlen(x, x_dtype, x_fp8, x_scale, H, T, d, cu_seqlens, nseq, signs, per_tensor,
                             hip_stream) -> int:
    return load().attn_fp8_quantize_varlen(x, x_dtype, x_fp8, x_scale, H, T, d, cu_seqlens, nseq, signs,
                                           per_tensor, hip_stream)


def attn_strerror(code: int) -> str:
    return load().attn_strerror(code).decode()


# ---------------------------------------------------------------- torch front

def _check(rc: int):
    if rc != ATTN_OK:
        raise RuntimeError(attn_strerror(rc))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return ATTN_DT_F16
    if t.dtype == torch.bfloat16:
        return ATTN_DT_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return ATTN_DT_FP8_E4M3
    if t.dtype == torch.float32:
        return ATTN_DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(dev) -> int:
    import torch

    return torch.cuda.current_stream(dev).cuda_stream


def forward(q, k, v, *, causal: bool = False, scale: Optional[float] = None, cu_seqlens_q=None,
            cu_seqlens_k=None, q_scale=None, k_scale=None, v_scale=None, out=None, lse=None):
    """Exact attention forward through ``attn_fwd_stream``.

    Dense: q [B, H, Nq, d], k/v [B, H, Nk, d] -> (o [B, H, Nq, d], lse [B, H, Nq]).
    Varlen (cu_seqlens_q/k int32 [B+1] on the device): q [H, Tq, d],
    k/v [H, Tk, d] -> (o [H, Tq, d], lse [H, Tq]).
    fp8 (q, k, v uint8 e4m3 codes with fp32 scales [B, H, ceil(N/128)], or
    for varlen [H, ceil(T/128) + B] as ``fp8_quantize_varlen`` writes them):
    o is bfloat16.  Tensors must be contiguous and on one GPU.
    """
    import torch

    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt or dt == ATTN_DT_F32:
        raise TypeError("q, k, v must share one of float16, bfloat16, uint8 (e4m3)")
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    varlen = cu_seqlens_q is not None
    if varlen:
        if q.dim() != 3:
            raise ValueError("varlen q must be [H, T, d]")
        H, Nq, _ = q.shape
        Nk = k.shape[1]
        B = cu_seqlens_q.numel() - 1
        lse_shape = (H, Nq)
    else:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, H, N, d]")
        B, H, Nq, _ = q.shape
        Nk = k.shape[2]
        lse_shape = (B, H, Nq)
    o_dtype = torch.bfloat16 if dt == ATTN_DT_FP8_E4M3 else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    rc = attn_fwd_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                         int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), dt,
                         _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _stream(q.device))
    _check(rc)
    return out, lse


def default_splits(B: int, H: int, Nq: int, Nk: int, rows_per_workgroup: int = 128,
                   target_workgroups: int = 512, min_keys: int = 512) -> int:
    """Key chunks for ``forward_splitkv``: about ``target_workgroups`` work
    items (two per compute unit: the key-chunk launches run two workgroups
    per CU; more chunks only add partial traffic and per-item overhead,
    measured), without chunks shorter than ``min_keys``."""
    items = B * H * max(1, -(-Nq // rows_per_workgroup))
    want = max(1, -(-target_workgroups // items))
    return int(max(1, min(want, Nk // min_keys if Nk >= min_keys else 1, 1024)))


def forward_splitkv(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                    num_splits: Optional[int] = None, out=None, lse=None, o_part=None, lse_part=None):
    """Attention over key chunks plus the merge, through ``attn_fwd_splitkv``.

    Dense fp16/bf16 only: q [B, H, Nq, d], k/v [B, H, Nk, d] -> (o, lse).
    ``o_part`` float32 [S, B, H, Nq, d] and ``lse_part`` float32 [S, B, H, Nq]
    are the workspace (allocated here if not given; they hold the per-chunk
    results afterwards).
    """
    import torch

    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = default_splits(B, H, Nq, Nk, target_workgroups=2 * cus)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if o_part is None:
        o_part = torch.empty((num_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((num_splits, B, H, Nq), dtype=torch.float32, device=q.device)
    if o_part.numel() < num_splits * B * H * Nq * d or lse_part.numel() < num_splits * B * H * Nq:
        raise ValueError("o_part / lse_part are smaller than num_splits chunks")
    rc = attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                          int(bool(causal)), dt, int(num_splits), _ptr(o_part), _ptr(lse_part),
                          _stream(q.device))
    _check(rc)
    return out, lse


def forward_splitkv_fp8(q8, q_scale, k8, k_scale, v8, v_scale, *, causal: bool = False,
                        scale: Optional[float] = None, num_splits: Optional[int] = None, out=None, lse=None,
                        o_part=None, lse_part=None):
    """fp8 attention over key chunks plus the merge, through
    ``attn_fwd_splitkv_fp8``: e4m3 codes (uint8) q8 [B, H, Nq, d], k8/v8
    [B, H, Nk, d] with their per-128-row-tile scales (as ``fp8_quantize``
    writes them) -> (o bfloat16, lse).  Workspace as ``forward_splitkv``."""
    import torch

    for t in (q8, k8, v8, q_scale, k_scale, v_scale):
        if not t.is_contiguous():
            raise ValueError("codes and scales must be contiguous")
    if any(_dtype_code(t) != ATTN_DT_FP8_E4M3 for t in (q8, k8, v8)):
        raise TypeError("q8, k8, v8 must be uint8 e4m3 codes")
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, Nq, d = q8.shape
    Nk = k8.shape[2]
    if q_scale.numel() < B * H * ((Nq + 127) // 128) or min(k_scale.numel(), v_scale.numel()) < B * H * (
            (Nk + 127) // 128):
        raise ValueError("scales must hold one entry per (b, h, 128-row tile)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q8.device).multi_processor_count
        num_splits = default_splits(B, H, Nq, Nk, target_workgroups=2 * cus)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q8.device)
    if o_part is None:
        o_part = torch.empty((num_splits, B, H, Nq, d), dtype=torch.float32, device=q8.device)
    if lse_part is None:
        lse_part = torch.empty((num_splits, B, H, Nq), dtype=torch.float32, device=q8.device)
    if o_part.numel() < num_splits * B * H * Nq * d or lse_part.numel() < num_splits * B * H * Nq:
        raise ValueError("o_part / lse_part are smaller than num_splits chunks")
    rc = attn_fwd_splitkv_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale), _ptr(out),
                              _ptr(lse), B, H, Nq, Nk, d, float(scale), int(bool(causal)), int(num_splits),
                              _ptr(o_part), _ptr(lse_part), _stream(q8.device))
    _check(rc)
    return out, lse


def forward_splitkv_noalloc(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                            num_splits: Optional[int] = None, out=None, lse=None):
    """``forward_splitkv`` through ``attn_fwd_splitkv_noalloc``: the per-chunk
    partials go to the library's fixed device scratch, so with ``out`` and
    ``lse`` given nothing is allocated.  Raises if the call exceeds the
    scratch (ATTN_ERR_TOO_LARGE)."""
    import torch

    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = default_splits(B, H, Nq, Nk, target_workgroups=2 * cus)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    rc = attn_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                                  int(bool(causal)), dt, int(num_splits), _stream(q.device))
    _check(rc)
    return out, lse


def forward_paged(q, k_cache, v_cache, block_table, seqlens_k, *, scale: Optional[float] = None,
                  k_scale=None, v_scale=None, kv_dtype: Optional[str] = None, num_splits: Optional[int] = None,
                  out=None, lse=None, o_part=None, lse_part=None):
    """Non-causal attention of q [B, H, Nq, d] over a paged cache through
    ``attn_fwd_paged``: k_cache, v_cache [num_pages, page_size, H, d],
    block_table int32 [B, max_pages], seqlens_k int32 [B] (all on the GPU)
    -> (o, lse).  The caches have q's dtype, or hold 8-bit codes (uint8;
    ``kv_dtype`` "e4m3" or "int8") with float32 ``k_scale`` / ``v_scale``
    [num_pages, page_size, H].  ``num_splits`` defaults to
    ``default_splits`` for the longest possible sequence."""
    import torch

    for t in (q, k_cache, v_cache, block_table, seqlens_k):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dt = _dtype_code(q)
    if kv_dtype is None:
        if _dtype_code(k_cache) != dt or _dtype_code(v_cache) != dt:
            raise TypeError("q and the caches must share one dtype")
        kvd = dt
    else:
        kvd = {"e4m3": ATTN_DT_FP8_E4M3, "int8": ATTN_DT_INT8}[kv_dtype]
        if k_cache.element_size() != 1 or v_cache.element_size() != 1 or k_scale is None or v_scale is None:
            raise TypeError("8-bit caches need 1-byte codes and k_scale / v_scale")
        for t in (k_scale, v_scale):
            if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(k_cache.shape[:3]):
                raise ValueError("k_scale / v_scale must be contiguous float32 [num_pages, page_size, H]")
    if block_table.dtype != torch.int32 or seqlens_k.dtype != torch.int32:
        raise TypeError("block_table and seqlens_k must be int32")
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, H, Nq, d] and the caches [num_pages, page_size, H, d]")
    B, H, Nq, d = q.shape
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape[2:]) != (H, d) or block_table.dim() != 2 or block_table.shape[0] != B or \
            tuple(seqlens_k.shape) != (B,):
        raise ValueError("cache / block_table / seqlens_k shapes do not match q")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = default_splits(B, H, Nq, max_pages * page_size, target_workgroups=2 * cus)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if o_part is None:
        o_part = torch.empty((num_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((num_splits, B, H, Nq), dtype=torch.float32, device=q.device)
    if o_part.numel() < num_splits * B * H * Nq * d or lse_part.numel() < num_splits * B * H * Nq:
        raise ValueError("o_part / lse_part are smaller than num_splits chunks")
    rc = attn_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                        _ptr(seqlens_k), _ptr(out), _ptr(lse), B, H, Nq, d, num_pages, page_size, max_pages,
                        float(scale), dt, kvd, int(num_splits), _ptr(o_part), _ptr(lse_part), _stream(q.device))
    _check(rc)
    return out, lse


def forward_paged_fp8(q8, q_scale, k_cache, v_cache, block_table, seqlens_k, *, k_scale, v_scale, kv_dtype: str,
                      scale: Optional[float] = None, num_splits: Optional[int] = None, out=None, lse=None,
                      o_part=None, lse_part=None):
    """Decoding attention of e4m3 queries q8 (uint8 codes [B, H, Nq, d],
    Nq <= 2) with q_scale float32 [B, H] over an 8-bit paged cache
    (``kv_dtype`` "e4m3" or "int8", scales as ``forward_paged``) through
    ``attn_fwd_paged_fp8`` -> (o bfloat16 [B, H, Nq, d], lse)."""
    import torch

    for t in (q8, q_scale, k_cache, v_cache, block_table, seqlens_k, k_scale, v_scale):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if q8.element_size() != 1 or k_cache.element_size() != 1 or v_cache.element_size() != 1:
        raise TypeError("q8 and the caches must hold 1-byte codes")
    kvd = {"e4m3": ATTN_DT_FP8_E4M3, "int8": ATTN_DT_INT8}[kv_dtype]
    if q8.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q8 must be [B, H, Nq, d] and the caches [num_pages, page_size, H, d]")
    B, H, Nq, d = q8.shape
    if q_scale.dtype != torch.float32 or tuple(q_scale.shape) != (B, H):
        raise ValueError("q_scale must be float32 [B, H]")
    for t in (k_scale, v_scale):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(k_cache.shape[:3]):
            raise ValueError("k_scale / v_scale must be float32 [num_pages, page_size, H]")
    if block_table.dtype != torch.int32 or seqlens_k.dtype != torch.int32:
        raise TypeError("block_table and seqlens_k must be int32")
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape[2:]) != (H, d) or block_table.dim() != 2 or block_table.shape[0] != B or \
            tuple(seqlens_k.shape) != (B,):
        raise ValueError("cache / block_table / seqlens_k shapes do not match q8")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q8.device).multi_processor_count
        num_splits = default_splits(B, H, Nq, max_pages * page_size, target_workgroups=2 * cus)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q8.device)
    if o_part is None:
        o_part = torch.empty((num_splits, B, H, Nq, d), dtype=torch.float32, device=q8.device)
    if lse_part is None:
        lse_part = torch.empty((num_splits, B, H, Nq), dtype=torch.float32, device=q8.device)
    if o_part.numel() < num_splits * B * H * Nq * d or lse_part.numel() < num_splits * B * H * Nq:
        raise ValueError("o_part / lse_part are smaller than num_splits chunks")
    rc = attn_fwd_paged_fp8(_ptr(q8), _ptr(q_scale), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                            _ptr(block_table), _ptr(seqlens_k), _ptr(out), _ptr(lse), B, H, Nq, d, num_pages,
                            page_size, max_pages, float(scale), kvd, int(num_splits), _ptr(o_part), _ptr(lse_part),
                            _stream(q8.device))
    _check(rc)
    return out, lse


def merge(o_part, lse_part, *, out_dtype=None, out=None, lse=None):
    """Combine per-chunk results: o_part float32 [S, B, H, Nq, d], lse_part
    float32 [S, B, H, Nq] -> (o [B, H, Nq, d] of ``out_dtype``, lse [B, H, Nq])."""
    import torch

    if o_part.dim() != 5 or lse_part.dim() != 4 or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("o_part must be a contiguous [S, B, H, Nq, d] and lse_part [S, B, H, Nq] tensor")
    S, B, H, Nq, d = o_part.shape
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=o_part.device)
    rc = attn_merge(_ptr(o_part), _ptr(lse_part), S, B, H, Nq, d, _ptr(out), _ptr(lse), _dtype_code(out),
                    _stream(o_part.device))
    _check(rc)
    return out, lse


def backward(q, k, v, o, lse, dout, *, causal: bool = False, scale: Optional[float] = None, cu_seqlens_q=None,
             cu_seqlens_k=None, dq=None, dk=None, dv=None, delta=None):
    """Gradients (dq, dk, dv) of ``forward(q, k, v)`` for the output gradient
    ``dout``, through ``attn_bwd``.  fp16/bf16, d = 64, 128 or 256.  Dense:
    q, o, dout [B, H, Nq, d]; k, v [B, H, Nk, d]; lse float32 [B, H, Nq] from
    the forward.  Varlen (cu_seqlens_q/k int32 [B+1] on the device):
    q, o, dout [H, Tq, d], k, v [H, Tk, d], lse [H, Tq].  ``delta`` float32
    (the shape of lse) is the workspace (allocated here if not given; it
    holds rowsum(dout * o) afterwards)."""
    import torch

    for t in (q, k, v, o, dout, lse):
        if not t.is_contiguous():
            raise ValueError("q, k, v, o, dout, lse must be contiguous")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share one dtype")
    varlen = cu_seqlens_q is not None
    nd = 3 if varlen else 4
    if q.dim() != nd or k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, o, dout must be [B, H, Nq, d] ([H, Tq, d] varlen) and k, v alike")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:-1]):
        raise ValueError("lse must be float32 with the shape of q without its last axis")
    if varlen:
        H, Nq, d = q.shape
        Nk = k.shape[1]
        B = cu_seqlens_q.numel() - 1
    else:
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty(tuple(lse.shape), dtype=torch.float32, device=q.device)
    rc = attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                  _ptr(delta), B, H, Nq, Nk, d, float(scale), int(bool(causal)), _ptr(cu_seqlens_q),
                  _ptr(cu_seqlens_k), dt, _stream(q.device))
    _check(rc)
    return dq, dk, dv


def backward_fp8(q8, q_scale, k8, k_scale, v8, v_scale, o, lse, dout, *, causal: bool = False,
                 scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) in bfloat16 of the fp8 ``forward`` on the e4m3
    codes q8, k8, v8 (uint8 [B, H, N, 128]) with their tile scales (float32
    [B, H, ceil(N/128)]), for the output gradient ``dout`` (bfloat16, the
    shape of o), through ``attn_bwd_fp8``.  o (bfloat16) and lse are the
    forward's outputs.  ``workspace`` is an optional tuple (stats, do8,
    do_scale) of the shapes attn_bwd_fp8 states (allocated here if absent)."""
    import torch

    for t in (q8, k8, v8, q_scale, k_scale, v_scale, o, lse, dout):
        if not t.is_contiguous():
            raise ValueError("all inputs must be contiguous")
    if q8.dtype != torch.uint8 or k8.dtype != torch.uint8 or v8.dtype != torch.uint8:
        raise TypeError("q8, k8, v8 must be uint8 e4m3 codes")
    if o.dtype != torch.bfloat16 or dout.dtype != torch.bfloat16:
        raise TypeError("o and dout must be bfloat16")
    if q8.dim() != 4 or k8.shape != v8.shape or o.shape != q8.shape or dout.shape != q8.shape:
        raise ValueError("q8, o, dout must be [B, H, Nq, d] and k8, v8 [B, H, Nk, d]")
    B, H, Nq, d = q8.shape
    Nk = k8.shape[2]
    if tuple(q_scale.shape) != (B, H, (Nq + 127) // 128) or tuple(k_scale.shape) != (B, H, (Nk + 127) // 128) \
            or k_scale.shape != v_scale.shape:
        raise ValueError("scales must be [B, H, ceil(N/128)]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be float32 [B, H, Nq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device) if dq is None else dq
    dk = torch.empty(k8.shape, dtype=torch.bfloat16, device=q8.device) if dk is None else dk
    dv = torch.empty(v8.shape, dtype=torch.bfloat16, device=q8.device) if dv is None else dv
    if workspace is None:
        workspace = (torch.empty((3, B, H, Nq), dtype=torch.float32, device=q8.device),
                     torch.empty(q8.shape, dtype=torch.uint8, device=q8.device),
                     torch.empty((B, H, (Nq + 127) // 128), dtype=torch.float32, device=q8.device))
    stats, do8, do_scale = workspace
    if stats.numel() < 3 * B * H * Nq or do8.numel() < B * H * Nq * d or do_scale.numel() < B * H * ((Nq + 127) // 128):
        raise ValueError("workspace too small")
    rc = attn_bwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale), _ptr(o),
                      _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(stats), _ptr(do8), _ptr(do_scale),
                      B, H, Nq, Nk, d, float(scale), int(bool(causal)), _stream(q8.device))
    _check(rc)
    return dq, dk, dv


def fp8_quantize(x, signs=None, per_tensor: bool = False, out=None, scales=None):
    """Incoherent processing (if ``signs``) and e4m3 block quantisation of x [B, H, N, d].

    Returns ``(codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N/128)])``.
    """
    import torch

    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] tensor")
    B, H, N, d = x.shape
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, (N + 127) // 128), dtype=torch.float32, device=x.device)
    rc = attn_fp8_quantize(_ptr(x), _dtype_code(x), _ptr(out), _ptr(scales), B, H, N, d, _ptr(signs),
                           int(bool(per_tensor)), _stream(x.device))
    _check(rc)
    return out, scales


def fp8_quantize_varlen(x, cu_seqlens, signs=None, per_tensor: bool = False, out=None, scales=None):
    """``fp8_quantize`` of a packed batch x [H, T, d] (sequence b on tokens
    [cu_seqlens[b], cu_seqlens[b+1]), cu_seqlens int32 on the device), with
    the 128-row tiles restarting at every sequence.

    Returns ``(codes uint8 [H, T, d], scales float32 [H, ceil(T/128) + nseq])``
    in the layout ``forward`` reads for fp8 with cu_seqlens.
    """
    import torch

    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [H, T, d] tensor")
    H, T, d = x.shape
    nseq = cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((H, (T + 127) // 128 + nseq), dtype=torch.float32, device=x.device)
    rc = attn_fp8_quantize_varlen(_ptr(x), _dtype_code(x), _ptr(out), _ptr(scales), H, T, d, _ptr(cu_seqlens),
                                  nseq, _ptr(signs), int(bool(per_tensor)), _stream(x.device))
    _check(rc)
    return out, scales
