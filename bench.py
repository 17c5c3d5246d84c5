"""Attention-forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-detail]

Workload (one "step"): the dense bf16 problem B=2, H=16, Nq=Nk=8192, d=128,
scale 1/sqrt(128), non-causal, seeded N(0,1) inputs already resident in HBM,
one launch through the C ABI (attn_fwd_stream on torch's current stream).
value = FLOPs / (time per step), FLOPs = 4 B H Nq Nk d.

Prints ONE JSON line with the roofline of that kernel (algorithmic FLOPs /
its mean launch duration from HIP events on its stream, against the dense
bf16 MFMA peak of 2.5 PFLOP/s; also against the MFMA rate a register-only
probe kernel sustains on this GPU) and the CPU baseline (the fp64 oracle,
timed on a bounded sample of the same workload: some of its heads).
"detail" adds the other shapes (B2 H16 N4096 d128 non-causal and causal,
d=256, variable length, the e4m3 kernel with its own roofline against the
fp8 peak of 5.0 PFLOP/s, decoding over key chunks, the backward pass), each
with its own TFLOP/s (or GB/s) and fraction of peak.  The detail rows run
before the timed step.

--copy-calib runs only a plain device copy of known size (for scaling the
HBM byte counters) and prints its byte count.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["exact_attention_forward_03_amd/csrc/attn_fwd.hip",
                  "exact_attention_forward_03_amd/csrc/attn_tile.h",
                  "exact_attention_forward_03_amd/csrc/attn_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_d128_n8192_traffic.json")
HEADLINE = "n8k_bf16"  # B2 H16 Nq=Nk=8192 d128 bf16 non-causal


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sample_heads: int = 8, chunk_heads: int = 2):
    """The fp64 oracle on a bounded sample of the headline workload: the
    first `sample_heads` of its B*H = 32 heads (seeded N(0,1) inputs rounded
    to bf16, then held in fp64 on the host), `chunk_heads` heads per oracle
    call to bound memory; generation excluded.  TFLOP/s uses the same FLOP
    count per head as the GPU line."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import workloads as W

    w = W.WORKLOADS[HEADLINE]
    rng = np.random.default_rng(0)
    shape = (sample_heads, w.Nq, w.d)
    q, k, v = (W.to_dtype(rng.standard_normal(shape, dtype=np.float32), "bf16").double().numpy() for _ in range(3))
    t0 = time.perf_counter()
    for h in range(0, sample_heads, chunk_heads):
        sl = slice(h, h + chunk_heads)
        oracle.attention(q[sl], k[sl], v[sl], w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = 4.0 * sample_heads * w.Nq * w.Nk * w.d
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] + [1])
    vendor = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas) or "unknown"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{sample_heads} of the {w.B * w.H} heads of the B2 H16 N8192 d128 bf16 non-causal workload "
                      f"(inputs in fp64), {chunk_heads} heads per oracle call, {dt:.1f} s",
            "cpu_model": _cpu_model(), "blas": vendor, "blas_threads": int(threads)}


def measured_mfma_tflops():
    """Dense MFMA rates measured by the probe library on this GPU, TFLOP/s:
    (bf16, fp8) on constant operands and (bf16, fp8) on random operand bits
    (the chip lowers its clock under the power of switching bits, so the
    second pair is what real data can reach); Nones if the probe is not
    built."""
    import ctypes

    path = os.path.join(ROOT, "exact_attention_forward_03_amd", "libattn_probe.so")
    if not os.path.exists(path):
        return None, None, None, None
    lib = ctypes.CDLL(path)
    lib.attn_probe_mfma_tflops.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.attn_probe_mfma_tflops.restype = ctypes.c_int
    out = []
    for kind in (0, 1, 2, 3):
        v = ctypes.c_double(0.0)
        rc = lib.attn_probe_mfma_tflops(kind, ctypes.byref(v), None)
        out.append(round(v.value, 1) if rc == 0 else None)
    return tuple(out)


def timed_launches(fn, n, stream):
    """Run fn() n times; return per-launch durations (ms) from events on `stream`."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def bench_one(attn, name, steps, warmup):
    """Mean and median launch time of one fp16/bf16 workload (seeded inputs
    resident in HBM, launches on torch's current stream)."""
    import numpy as np
    import torch

    import workloads as W

    stream = torch.cuda.current_stream()
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    q, k, v = (W.to_dtype(x[n], w.dtype).cuda() for n in ("q", "k", "v"))
    kw = {}
    if w.varlen:
        cu = torch.from_numpy(x["cu_seqlens"]).cuda()
        kw = dict(cu_seqlens_q=cu, cu_seqlens_k=cu)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

    def run():
        attn.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, **kw)

    for _ in range(warmup):
        run()
    ts = timed_launches(run, steps, stream)
    ms, med = float(np.mean(ts)), float(np.median(ts))
    tf = w.flops() / (ms / 1e3) / 1e12
    return {"ms": round(ms, 4), "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "ms_median": round(med, 4), "tflops_median": round(w.flops() / (med / 1e3) / 1e12, 2),
            "causal": w.causal, "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}


DETAIL_WARMUP = 100  # untimed launches per detail shape, at least (new inputs: ~100 to settle)


def bench_detail(attn, steps, warmup):
    """Per-shape throughput of the other workloads (mean and median over
    `steps` launches, after at least DETAIL_WARMUP untimed ones)."""
    warmup = max(warmup, DETAIL_WARMUP)
    out = {}
    for name in ("dense_bf16", "dense_bf16_causal", "hdim256_bf16", "varlen_bf16_causal", "tiny_f16"):
        out[name] = bench_one(attn, name, steps, warmup)
    out["hbm_copy_gbs"] = copy_bandwidth()
    out.update(bench_decode(attn, steps, warmup))
    out.update(bench_backward(attn, steps, warmup))
    fp8 = bench_fp8(attn, steps, warmup)
    if fp8:
        out.update(fp8)
    return out


def bench_decode(attn, steps, warmup):
    """Decoding (B=2 H=32, one query per head, Nk=32768, d=128, bf16): attention
    over key chunks plus the merge, against HBM bandwidth (the K and V bytes
    are the algorithmic traffic); the single-pass kernel on the same shape
    for comparison; the same keys and values read from a paged cache, and a
    paged cache of e4m3 codes with per-(token, head) scales (bytes: codes and
    scales), read by bf16 and by e4m3 queries."""
    import numpy as np
    import torch

    import workloads as W

    w = W.WORKLOADS["decode_bf16"]
    x = W.make_inputs(w)
    q, k, v = (W.to_dtype(x[n], w.dtype).cuda() for n in ("q", "k", "v"))
    splits = attn.default_splits(w.B, w.H, w.Nq, w.Nk,
                                 target_workgroups=2 * torch.cuda.get_device_properties(0).multi_processor_count)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    op = torch.empty((splits,) + tuple(q.shape), dtype=torch.float32, device="cuda")
    lp = torch.empty((splits,) + tuple(q.shape[:-1]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def run_split():
        attn.forward_splitkv(q, k, v, scale=w.scale, num_splits=splits, out=o, lse=lse, o_part=op, lse_part=lp)

    def run_single():
        attn.forward(q, k, v, scale=w.scale, out=o, lse=lse)

    for _ in range(warmup):
        run_split()
        run_single()
    ms = float(np.mean(timed_launches(run_split, steps, stream)))
    ms1 = float(np.mean(timed_launches(run_single, steps, stream)))
    kv_bytes = 2 * k.numel() * 2
    gbs = kv_bytes / (ms / 1e3) / 1e9
    out = {"decode_bf16_splitkv": {"ms": round(ms, 4), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                   "num_splits": splits, "single_pass_ms": round(ms1, 4),
                                   "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}}

    # the same keys and values in a paged cache: 256-token pages stored in a
    # shuffled order, read through the page table
    P = 256
    n_pages = w.B * w.Nk // P
    perm = torch.from_numpy(np.random.default_rng(1).permutation(n_pages)).cuda()
    kc = torch.empty((n_pages, P, w.H, w.d), dtype=k.dtype, device="cuda")
    vc = torch.empty_like(kc)
    kc[perm] = k.transpose(1, 2).reshape(n_pages, P, w.H, w.d)
    vc[perm] = v.transpose(1, 2).reshape(n_pages, P, w.H, w.d)
    table = perm.to(torch.int32).reshape(w.B, w.Nk // P).contiguous()
    lens = torch.full((w.B,), w.Nk, dtype=torch.int32, device="cuda")

    def run_paged():
        attn.forward_paged(q, kc, vc, table, lens, scale=w.scale, num_splits=splits, out=o, lse=lse, o_part=op,
                           lse_part=lp)

    for _ in range(warmup):
        run_paged()
    msp = float(np.mean(timed_launches(run_paged, steps, stream)))
    gbp = kv_bytes / (msp / 1e3) / 1e9
    out["decode_bf16_paged"] = {"ms": round(msp, 4), "gbs": round(gbp, 1), "frac_hbm": round(gbp / HBM_PEAK_GBS, 4),
                                "page_size": P, "num_splits": splits, "vs_contiguous": round(msp / ms, 4),
                                "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}

    # an e4m3 cache of the same shape (random codes, per-(token, head) scales)
    k8 = torch.from_numpy(W.random_e4m3_codes(tuple(kc.shape), 2)).cuda()
    v8 = torch.from_numpy(W.random_e4m3_codes(tuple(kc.shape), 3)).cuda()
    ks = torch.from_numpy(W.random_scales(tuple(kc.shape[:3]), 4)).cuda()
    vs = torch.from_numpy(W.random_scales(tuple(kc.shape[:3]), 5)).cuda()
    del kc, vc

    def run_paged8():
        attn.forward_paged(q, k8, v8, table, lens, scale=w.scale, k_scale=ks, v_scale=vs, kv_dtype="e4m3",
                           num_splits=splits, out=o, lse=lse, o_part=op, lse_part=lp)

    for _ in range(warmup):
        run_paged8()
    ms8 = float(np.mean(timed_launches(run_paged8, steps, stream)))
    b8 = 2 * (k8.numel() + ks.numel() * 4)
    gb8 = b8 / (ms8 / 1e3) / 1e9
    out["decode_e4m3_paged"] = {"ms": round(ms8, 4), "gbs": round(gb8, 1), "frac_hbm": round(gb8 / HBM_PEAK_GBS, 4),
                                "page_size": P, "num_splits": splits, "vs_bf16_paged": round(ms8 / msp, 4),
                                "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}

    # the same cache with e4m3 queries (one scale per batch and head)
    q8 = torch.from_numpy(W.random_e4m3_codes(tuple(q.shape), 6)).cuda()
    qs = torch.from_numpy(W.random_scales((w.B, w.H), 7, 0.5, 2.0)).cuda()
    o8 = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

    def run_paged8q():
        attn.forward_paged_fp8(q8, qs, k8, v8, table, lens, scale=w.scale, k_scale=ks, v_scale=vs, kv_dtype="e4m3",
                               num_splits=splits, out=o8, lse=lse, o_part=op, lse_part=lp)

    for _ in range(warmup):
        run_paged8q()
    ms8q = float(np.mean(timed_launches(run_paged8q, steps, stream)))
    gb8q = b8 / (ms8q / 1e3) / 1e9
    out["decode_e4m3q_e4m3_paged"] = {"ms": round(ms8q, 4), "gbs": round(gb8q, 1),
                                      "frac_hbm": round(gb8q / HBM_PEAK_GBS, 4), "page_size": P,
                                      "num_splits": splits, "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}
    return out


def bench_backward(attn, steps, warmup):
    """Backward pass (attn_bwd: delta, dK/dV and dQ kernels) on the dense
    bf16 shape B=2 H=16 N=4096 d=128, non-causal and causal, and on the
    large-head shape B=1 H=16 N=8192 d=256 (non-causal).  FLOPs are those
    of the five products of the gradient (S, dP, dV, dK, dQ: 10 B H N^2 d,
    halved for causal); the kernels recompute S and dP once more for dQ.
    The d=128 shapes are also run through attn_bwd_fp8 (e4m3 inputs from
    attn_fp8_quantize, E5M2 gradient operands), priced against the fp8
    peak with the same FLOP count."""
    import numpy as np
    import torch

    import workloads as W

    out = {}
    stream = torch.cuda.current_stream()
    for name in ("dense_bf16", "dense_bf16_causal", "hdim256_bf16"):
        w = W.WORKLOADS[name]
        rng = np.random.default_rng(5)
        shape = (w.B, w.H, w.Nq, w.d)
        q, k, v, do = (W.to_dtype(rng.standard_normal(shape, dtype=np.float32), "bf16").cuda() for _ in range(4))
        o, lse = attn.forward(q, k, v, causal=w.causal, scale=w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

        def run():
            attn.backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, delta=delta)

        for _ in range(warmup):
            run()
        ms = float(np.mean(timed_launches(run, steps, stream)))
        flops = 10.0 * w.B * w.H * w.Nq * w.Nk * w.d * (0.5 if w.causal else 1.0)
        tf = flops / (ms / 1e3) / 1e12
        out["bwd_" + name] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                              "causal": w.causal, "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}
        if w.d == 128:
            # the same shape on e4m3 operands with E5M2 gradients (attn_bwd_fp8)
            q8, sq = attn.fp8_quantize(q)
            k8, sk = attn.fp8_quantize(k)
            v8, sv = attn.fp8_quantize(v)
            o8, lse8 = attn.forward(q8, k8, v8, causal=w.causal, scale=w.scale, q_scale=sq, k_scale=sk,
                                    v_scale=sv)
            ws = (torch.empty((3,) + tuple(q.shape[:-1]), dtype=torch.float32, device="cuda"),
                  torch.empty(q.shape, dtype=torch.uint8, device="cuda"),
                  torch.empty(tuple(q.shape[:-2]) + ((w.Nq + 127) // 128,), dtype=torch.float32, device="cuda"))

            def run8():
                attn.backward_fp8(q8, sq, k8, sk, v8, sv, o8, lse8, do, causal=w.causal, scale=w.scale, dq=dq,
                                  dk=dk, dv=dv, workspace=ws)

            for _ in range(warmup):
                run8()
            ms8 = float(np.mean(timed_launches(run8, steps, stream)))
            tf8 = flops / (ms8 / 1e3) / 1e12
            out["bwd_fp8_" + name.replace("_bf16", "")] = {
                "ms": round(ms8, 4), "tflops": round(tf8, 2), "frac": round(tf8 / PEAK_FP8_TFLOPS, 4),
                "vs_bf16": round(ms8 / ms, 4), "causal": w.causal, "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}
            del q8, k8, v8, o8, lse8, ws
        del q, k, v, do, o, lse, dq, dk, dv, delta
    return out


def copy_bandwidth(steps: int = 10) -> float:
    """GB/s (bytes read + written) of a plain 1 GiB device-to-device copy:
    the HBM rate a streaming kernel reaches on this GPU, next to the spec
    peak, for the memory-bound rows."""
    import numpy as np
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    ms = float(np.mean(timed_launches(lambda: b.copy_(a), steps, torch.cuda.current_stream())))
    del a, b
    return round(2 * n / (ms / 1e3) / 1e9, 1)


def bench_fp8(attn, steps, warmup, varlen=True, extras=True):
    """fp8 workload (B=2 H=16 N=8192 d=128, outlier channels): the attention
    kernel alone and the pre-processing of Q, K, V; None if not built."""
    import numpy as np
    import torch

    import workloads as W

    w = W.WORKLOADS["fp8_outlier"]
    x = W.make_inputs(w)
    q32, k32, v32 = (torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v"))
    signs = torch.from_numpy(x["signs"]).cuda()
    try:
        q8, sq = attn.fp8_quantize(q32, signs)
        k8, sk = attn.fp8_quantize(k32, signs)
        v8, sv = attn.fp8_quantize(v32, None)
        o, lse = attn.forward(q8, k8, v8, scale=w.scale, q_scale=sq, k_scale=sk, v_scale=sv)
    except RuntimeError:
        return None
    stream = torch.cuda.current_stream()

    def run_attn():
        attn.forward(q8, k8, v8, scale=w.scale, q_scale=sq, k_scale=sk, v_scale=sv, out=o, lse=lse)

    def run_prep():
        attn.fp8_quantize(q32, signs, out=q8, scales=sq)
        attn.fp8_quantize(k32, signs, out=k8, scales=sk)
        attn.fp8_quantize(v32, None, out=v8, scales=sv)

    for _ in range(warmup):
        run_attn()
        run_prep()
    ts = timed_launches(run_attn, steps, stream)
    ms, med = float(np.mean(ts)), float(np.median(ts))
    ms_prep = float(np.mean(timed_launches(run_prep, steps, stream)))
    tf = w.flops() / (ms / 1e3) / 1e12
    prep_bytes = 3 * q32.numel() * (4 + 1) + 3 * sq.numel() * 4
    return {"fp8_outlier": {"ms": round(ms, 4), "tflops": round(tf, 2), "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                            "ms_median": round(med, 4),
                            "tflops_median": round(w.flops() / (med / 1e3) / 1e12, 2),
                            "shape": [w.B, w.H, w.Nq, w.Nk, w.d],
                            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                                         "kernel": "attn_fwd_fp8_kernel<d=128, 128-key tiles, non-causal, 4 waves, 2 slots>",
                                         "mean_launch_ms": round(ms, 4)}},
            "fp8_prep_qkv": {"ms": round(ms_prep, 4), "gbs": round(prep_bytes / (ms_prep / 1e3) / 1e9, 1),
                             "frac_hbm": round(prep_bytes / (ms_prep / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
            # fp32 Q, K, V in HBM -> rotation and block quantisation -> e4m3 attention
            "fp8_end_to_end": {"ms": round(ms + ms_prep, 4),
                               "tflops": round(w.flops() / ((ms + ms_prep) / 1e3) / 1e12, 2)},
            **(bench_fp8_hdim256(attn, steps, warmup) if extras else {}),
            **(bench_fp8_splitkv(attn, steps, warmup) if extras else {}),
            **(bench_fp8_varlen(attn, steps, warmup) if varlen and extras else {})}


def bench_fp8_hdim256(attn, steps, warmup):
    """The large-head shape (B=1 H=16 N=8192 d=256, N(0,1), non-causal) in
    fp8: Q, K rotated and block-quantised, V block-quantised on the device,
    then the e4m3 attention kernel alone is timed (64-key tiles at d=256)."""
    import numpy as np
    import torch

    import workloads as W

    w = W.WORKLOADS["hdim256_bf16"]
    x = W.make_inputs(w)
    signs = torch.from_numpy(np.random.default_rng(w.seed).choice([-1.0, 1.0], w.d).astype(np.float32)).cuda()
    q8, sq = attn.fp8_quantize(torch.from_numpy(x["q"]).cuda(), signs)
    k8, sk = attn.fp8_quantize(torch.from_numpy(x["k"]).cuda(), signs)
    v8, sv = attn.fp8_quantize(torch.from_numpy(x["v"]).cuda(), None)
    o, lse = attn.forward(q8, k8, v8, scale=w.scale, q_scale=sq, k_scale=sk, v_scale=sv)
    stream = torch.cuda.current_stream()

    def run():
        attn.forward(q8, k8, v8, scale=w.scale, q_scale=sq, k_scale=sk, v_scale=sv, out=o, lse=lse)

    for _ in range(warmup):
        run()
    ms = float(np.mean(timed_launches(run, steps, stream)))
    tf = w.flops() / (ms / 1e3) / 1e12
    return {"fp8_hdim256": {"ms": round(ms, 4), "tflops": round(tf, 2), "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                            "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}}


def bench_fp8_splitkv(attn, steps, warmup):
    """Long keys and few query tiles in fp8 (B=1 H=16 Nq=512 Nk=65536 d=128,
    N(0,1), non-causal): the e4m3 kernel over 8 key chunks plus the merge
    (attn_fwd_splitkv_fp8), beside the one-pass kernel on the same codes."""
    import numpy as np
    import torch

    B, H, nq, nk, d = 1, 16, 512, 65536, 128
    g = torch.Generator().manual_seed(11)
    q8, sq = attn.fp8_quantize(torch.randn(B, H, nq, d, generator=g).cuda())
    k8, sk = attn.fp8_quantize(torch.randn(B, H, nk, d, generator=g).cuda())
    v8, sv = attn.fp8_quantize(torch.randn(B, H, nk, d, generator=g).cuda())
    scale = 1.0 / np.sqrt(d)
    stream = torch.cuda.current_stream()
    o = torch.empty(B, H, nq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, nq, dtype=torch.float32, device="cuda")
    S = 8
    op = torch.empty(S, B, H, nq, d, dtype=torch.float32, device="cuda")
    lp = torch.empty(S, B, H, nq, dtype=torch.float32, device="cuda")

    def split():
        attn.forward_splitkv_fp8(q8, sq, k8, sk, v8, sv, scale=scale, num_splits=S, out=o, lse=lse, o_part=op,
                                 lse_part=lp)

    def one_pass():
        attn.forward(q8, k8, v8, scale=scale, q_scale=sq, k_scale=sk, v_scale=sv, out=o, lse=lse)

    flops = 4.0 * B * H * nq * nk * d
    out = {}
    for name, fn in (("fp8_splitkv_long_keys", split), ("fp8_one_pass_long_keys", one_pass)):
        for _ in range(warmup):
            fn()
        ms = float(np.mean(timed_launches(fn, steps, stream)))
        tf = flops / (ms / 1e3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 2), "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                     "shape": [B, H, nq, nk, d], "num_splits": S if fn is split else 1}
    return out


def bench_fp8_varlen(attn, steps, warmup):
    """The variable-length causal workload (8 sequences, H=32, d=128) in fp8:
    Q, K rotated and quantised per sequence tile on the device, then the
    e4m3 attention kernel alone is timed."""
    import numpy as np
    import torch

    import workloads as W

    w = W.WORKLOADS["varlen_bf16_causal"]
    x = W.make_inputs(w)
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    signs = torch.from_numpy(np.random.default_rng(w.seed).choice([-1.0, 1.0], w.d).astype(np.float32)).cuda()
    q8, sq = attn.fp8_quantize_varlen(torch.from_numpy(x["q"]).cuda(), cu, signs)
    k8, sk = attn.fp8_quantize_varlen(torch.from_numpy(x["k"]).cuda(), cu, signs)
    v8, sv = attn.fp8_quantize_varlen(torch.from_numpy(x["v"]).cuda(), cu, None)
    o, lse = attn.forward(q8, k8, v8, causal=True, scale=w.scale, cu_seqlens_q=cu, cu_seqlens_k=cu,
                          q_scale=sq, k_scale=sk, v_scale=sv)
    stream = torch.cuda.current_stream()

    def run():
        attn.forward(q8, k8, v8, causal=True, scale=w.scale, cu_seqlens_q=cu, cu_seqlens_k=cu,
                     q_scale=sq, k_scale=sk, v_scale=sv, out=o, lse=lse)

    for _ in range(warmup):
        run()
    ts = timed_launches(run, steps, stream)
    ms, med = float(np.mean(ts)), float(np.median(ts))
    tf = w.flops() / (ms / 1e3) / 1e12
    return {"fp8_varlen_causal": {"ms": round(ms, 4), "tflops": round(tf, 2), "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                                  "ms_median": round(med, 4),
                                  "tflops_median": round(w.flops() / (med / 1e3) / 1e12, 2),
                                  "shape": [w.B, w.H, w.Nq, w.Nk, w.d]}}


def copy_calib():
    """A plain copy of 1 GiB, to scale FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # a launch on newly allocated inputs runs up to ~15 % slower for its first
    # ~100 repetitions; the default warm-up covers that
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--only", default=None,
                    help="time one workload alone (a name of workloads.WORKLOADS, or fp8_outlier for the e4m3 "
                         "kernel) and print its own line: for profiling single kernels")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calib:
        copy_calib()
        return

    import exact_attention_forward_03_amd as attn
    import workloads as W

    attn.load()
    if args.only:
        if args.only == "fp8_outlier":
            res = bench_fp8(attn, args.steps, args.warmup, extras=False)["fp8_outlier"]
        else:
            res = bench_one(attn, args.only, args.steps, args.warmup)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return
    detail = None
    if not args.no_detail:
        detail = bench_detail(attn, max(10, args.steps // 2), 10)
    w = W.WORKLOADS[HEADLINE]
    x = W.make_inputs(w)
    q, k, v = (W.to_dtype(x[n], "bf16").cuda() for n in ("q", "k", "v"))
    del x
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        attn.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    step_ms = float(np.mean(ms))
    value = w.flops() / (step_ms / 1e3) / 1e12

    result = {
        "metric": "attention fwd TFLOP/s and % MFMA peak (bf16 + fp8), hdim 128/256, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense bf16 attention fwd, B=2 H=16 Nq=Nk=8192 d=128, non-causal",
                   "B": w.B, "H": w.H, "seq_len": w.Nq, "head_dim": w.d, "causal": w.causal,
                   "wall_s_timed": round(wall, 4), "ms_per_step_median": round(float(np.median(ms)), 4)},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": load_traffic(),
                     "kernel": "attn_fwd_dma_kernel<bf16, d=128, non-causal>, 512 workgroups of 512 threads",
                     "mean_launch_ms": round(step_ms, 4)},
    }
    mb16, mf8, rb16, rf8 = measured_mfma_tflops()
    result["roofline"]["measured_mfma_peak"] = mb16
    result["roofline"]["frac_of_measured_peak"] = round(value / mb16, 4) if mb16 else None
    result["roofline"]["measured_mfma_peak_random_operands"] = rb16
    result["roofline"]["frac_of_measured_peak_random_operands"] = round(value / rb16, 4) if rb16 else None
    if detail is not None:
        if mf8 and "fp8_outlier" in detail:
            fp8 = detail["fp8_outlier"]
            fp8["measured_mfma_peak"] = mf8
            fp8["frac_of_measured_peak"] = round(fp8["tflops"] / mf8, 4)
            fp8["measured_mfma_peak_random_operands"] = rf8
            fp8["frac_of_measured_peak_random_operands"] = round(fp8["tflops"] / rf8, 4) if rf8 else None
        result["detail"] = detail
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
