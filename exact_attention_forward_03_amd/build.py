"""Build ``libattn.so`` (the C ABI of include/attn.h) for gfx950 with hipcc,
and ``libattn_probe.so`` (the MFMA throughput probe that bench.py reports
next to the spec peak; not part of the attention ABI).

Every source is compiled to an object in ``_build/`` in parallel, then
linked into ``exact_attention_forward_03_amd/libattn.so`` and
``libattn_probe.so``.  Always rebuilds.

    python -m exact_attention_forward_03_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
PROBE_LIB = os.path.join(PKG, "libattn_probe.so")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_fp8.hip", "fp8_prep.hip", "attn_merge.hip", "attn_bwd.hip",
           "attn_bwd_fp8.hip", "attn_noalloc.hip", "attn_decode.hip"]
PROBE_SOURCES = ["mfma_peak.hip"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    flags = COMMON_FLAGS + list(extra_flags or [])
    procs = []
    objs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = [cc] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    n = len(SOURCES)
    for lib, lib_objs in ((LIB, objs[:n]), (PROBE_LIB, objs[n:])):
        tmp = lib + ".tmp"
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + lib_objs
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
