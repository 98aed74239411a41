"""Build libfa.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage:  python -m exact_tiled_attention_04_amd.build [-v]

Every call recompiles all sources (objects go to ``_build/`` at the repository
root) and atomically replaces ``exact_tiled_attention_04_amd/libfa.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd_mfma.hip", "fa_fwd_f32.hip", "fa_bwd_mfma.hip", "fa_fwd_fp8.hip", "fa_decode.hip"]

# Packed fp32 VALU instructions are kept out of every device code object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fno-honor-nans", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
