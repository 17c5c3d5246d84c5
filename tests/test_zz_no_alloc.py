"""GPU check of attn_fwd_splitkv_noalloc, the split-KV entry point whose
partial outputs live in the library's fixed device scratch instead of a
caller workspace, through the C ABI.

Two calls in a row (the second smaller, so it reuses the scratch that the
first left filled), each against attn_fwd_splitkv on the same inputs and
chunk count: the same kernels and chunks, so O and lse must be identical;
and against the fp64 oracle at the dense bars.  A call past the scratch
returns ATTN_ERR_TOO_LARGE and leaves the outputs untouched.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, to_device

pytestmark = pytest.mark.gpu


def _both(attn, B, H, nq, nk, d, dtype, causal, splits, seed):
    rng = np.random.default_rng(seed)
    qd, q64 = to_device(rng.standard_normal((B, H, nq, d), dtype=np.float32), dtype)
    kd, k64 = to_device(rng.standard_normal((B, H, nk, d), dtype=np.float32), dtype)
    vd, v64 = to_device(rng.standard_normal((B, H, nk, d), dtype=np.float32), dtype)
    dt = attn.ATTN_DT_F16 if dtype == "f16" else attn.ATTN_DT_BF16
    scale = 1.0 / np.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    o1 = torch.full_like(qd, float("nan"))
    l1 = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device="cuda")
    op = torch.empty((splits, B, H, nq, d), dtype=torch.float32, device="cuda")
    lp = torch.empty((splits, B, H, nq), dtype=torch.float32, device="cuda")
    rc = attn.attn_fwd_splitkv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(), l1.data_ptr(), B, H, nq,
                               nk, d, scale, int(causal), dt, splits, op.data_ptr(), lp.data_ptr(), stream)
    assert rc == attn.ATTN_OK
    o2 = torch.full_like(qd, float("nan"))
    l2 = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rc = attn.attn_fwd_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(), B,
                                       H, nq, nk, d, scale, int(causal), dt, splits, stream)
    assert rc == attn.ATTN_OK, attn.attn_strerror(rc)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = oracle.attention(q64, k64, v64, scale, causal)
    check(o2.double().cpu().numpy(), l2.double().cpu().numpy(), o_ref, l_ref, dtype,
          f"noalloc B{B} H{H} {nq}x{nk} d{d} {dtype} causal{causal} S{splits}")


def test_noalloc_matches_splitkv_twice(gpu_lib):
    # 2 * 8 * 300 * 6 = 28800 partial rows of 129 floats: 14.9 MB of the 32 MiB
    _both(gpu_lib, 2, 8, 300, 3000, 128, "bf16", True, 6, seed=3)
    _both(gpu_lib, 1, 3, 37, 500, 64, "f16", False, 3, seed=4)


def test_noalloc_too_large(gpu_lib):
    B, H, nq, nk, d, splits = 4, 32, 64, 256, 128, 16  # 131072 rows: 67.6 MB > 32 MiB
    q = torch.zeros((B, H, nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, nq), 7.0, dtype=torch.float32, device="cuda")
    rc = gpu_lib.attn_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(), B,
                                          H, nq, nk, d, 0.1, 0, gpu_lib.ATTN_DT_BF16, splits,
                                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == gpu_lib.ATTN_ERR_TOO_LARGE
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
