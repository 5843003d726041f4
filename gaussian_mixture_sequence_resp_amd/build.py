"""Builds libgma.so (HIP C++ for gfx950) in-tree with hipcc, and the benchmark's device peak
probe libgma_probe.so.

Flags: -O3 for gfx950 only; packed-fp32 VALU instructions are disabled for every
HIP translation unit (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgma.so")
SOURCES = ["gma_api.cpp", "gma_simt.hip", "gma_mfma.hip", "gma_mfma_causal.hip", "gma_causal_fused.hip", "gma_decode.hip", "gma_stats.hip", "gma_backward.hip",
           "gma_noalloc.hip"]
ARCH = "gfx950"
PROBE = "gma_probe.hip"
PROBE_LIB = os.path.join(HERE, "libgma_probe.so")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object in parallel, then link libgma.so."""
    from concurrent.futures import ThreadPoolExecutor

    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Wno-pass-failed", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(HERE, "..", "include")]
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if msgs and verbose:
            print("\n".join(msgs), file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], check=True)
    os.replace(tmp, LIB)
    # the benchmark's device peak probe, a library of its own (not part of the GMA ABI)
    pobj = compile_one(PROBE)
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", pobj, "-o", tmp], check=True)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
