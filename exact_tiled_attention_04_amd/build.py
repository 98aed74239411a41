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
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
# Device code may assume no NaN reaches its arithmetic (inputs are finite by
# contract); the host code's argument checks must see NaN as NaN, so it is
# compiled without this flag.
KERNEL_ONLY = ["-fno-honor-nans"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


# Host-side sanitizers for the checking build: AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (each flag behind
# -Xarch_host, so device code objects are built exactly as in the product).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link libfa.so in the package directory; with
    ``sanitize``, the same library with host-side sanitizers into
    ``_build/sanitize/libfa.so`` (loaded only by the sanitizer test, with the
    sanitizer runtime preloaded)."""
    cc = hipcc()
    build_dir = os.path.join(BUILD_DIR, "sanitize") if sanitize else BUILD_DIR
    lib_path = os.path.join(build_dir, "libfa.so") if sanitize else LIB_PATH
    san = SANITIZE_HOST if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = KERNEL_ONLY if src.endswith(".hip") else []
        cmd = [cc, *COMMON, *extra, *san, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
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
    tmp = lib_path + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path} in {time.time() - t0:.1f}s", flush=True)
    return lib_path


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_caller", "fa_c_caller.c")
C_CALLER_BIN = os.path.join(ROOT, "tests", "c_caller", "fa_c_caller")


def build_c_caller(verbose: bool = False) -> str:
    """Compile the plain C caller of the library (its GPU test runs it) with
    gcc as C99, against include/fa.h and the HIP runtime's C API, linked to
    the in-tree libfa.so (found through an rpath relative to the binary)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    gcc = shutil.which("gcc") or "gcc"
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(rocm, "include"), "-I", INCLUDE, C_CALLER_SRC, "-o", C_CALLER_BIN + ".tmp",
           "-L", PKG, "-lfa", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../exact_tiled_attention_04_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("C caller build failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(C_CALLER_BIN + ".tmp", C_CALLER_BIN)
    return C_CALLER_BIN


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize-host" in sys.argv)
    if "--sanitize-host" not in sys.argv:
        build_c_caller(verbose="-v" in sys.argv)
