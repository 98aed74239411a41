"""The C-ABI checks of ``tests/test_abi.py`` again, against a build of the
library whose host code runs under AddressSanitizer and
UndefinedBehaviorSanitizer (device code unchanged).  Host validation is the
part of the library a caller's bad arguments reach; any out-of-bounds access,
overflow, invalid enum or other undefined behaviour there aborts the run.
CPU only: no call in those tests reaches a kernel launch."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    clang = shutil.which("clang", path="/opt/rocm/llvm/bin")
    if clang is None:
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the library")
def test_abi_checks_under_host_sanitizers():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from exact_tiled_attention_04_amd.build import build
    lib = build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=runtime, FA_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
