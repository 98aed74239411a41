"""CPU checks of the C side of the boundary: include/fa.h on its own, and
the plain C caller with it, compile as ISO C99 with every warning an error
(gcc, no C++ or HIP compiler; the HIP runtime's headers are system headers)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="gcc and the HIP runtime headers are needed")
def test_c_caller_compiles_as_c99():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
                        "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                        "-fsyntax-only", os.path.join(ROOT, "tests", "c_caller", "fa_c_caller.c")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed")
def test_header_alone_is_iso_c(tmp_path):
    """fa.h needs no other header beyond the C standard library's."""
    src = tmp_path / "h.c"
    src.write_text('#include "fa.h"\nint main(void) { return fa_version() > 0 ? 0 : 1; }\n')
    for std in ("c99", "c11"):
        r = subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                            os.path.join(ROOT, "include"), "-fsyntax-only", str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
