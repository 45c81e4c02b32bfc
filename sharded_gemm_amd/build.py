"""Builds libtpshard.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sharded_gemm_amd.build          # or: __graft_entry__.build()

Sources are compiled to objects in parallel under ``_build/`` and linked
into ``sharded_gemm_amd/libtpshard.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libtpshard.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "checker.cpp", "api.cpp", "timing.cpp", "shard.hip", "reduce.hip", "gemm.hip", "noalloc.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 ALU ops in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 5) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
