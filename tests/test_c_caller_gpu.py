"""The library called from plain C (``tests/c_caller/fa_c_caller.c``: the
HIP runtime's C API for memory and a stream, then fa_fwd_bf16 and
fa_bwd_bf16, then two calls the library must refuse), its results checked
against the fp64 oracles at the bounds of the forward and backward parity
modules.  The binary is built with the library by ``__graft_entry__.build()``.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from oracle import attention_fwd
from tests.gpu_util import announce, compare
from tests.test_bwd_gpu import check_grads, oracle_grads
from workloads import random_grad, random_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_CALLER = os.path.join(ROOT, "tests", "c_caller", "fa_c_caller")

pytestmark = pytest.mark.gpu


def _bits(x):
    """float32 values exact in bfloat16 -> their 16-bit patterns."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _from_bits(path, shape):
    u = np.fromfile(path, dtype=np.uint16).reshape(shape)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("causal,wl", [(1, -1), (0, 100)])
def test_c_caller_matches_oracle(tmp_path, causal, wl):
    assert os.path.exists(C_CALLER), "tests/c_caller/fa_c_caller is not built (run __graft_entry__.build())"
    B, Hq, Hkv, N, d = 1, 4, 2, 333, 128
    scale = np.float32(d ** -0.5)
    q, k, v = random_inputs(8600 + causal, "bf16", B, Hq, Hkv, N, d)
    do = random_grad(8650 + causal, "bf16", B, Hq, N, d)
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        _bits(x).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "args.txt").write_text(f"{B} {Hq} {Hkv} {N} {d} {causal} {wl} {float(scale):.9g}\n")
    label = f"C caller B={B} H={Hq}/{Hkv} N={N} d={d} causal={causal} wl={wl}"
    announce(label)
    r = subprocess.run([C_CALLER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "fa_c_caller: ok" in r.stdout
    o = _from_bits(tmp_path / "o.bin", q.shape)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(B, Hq, N).astype(np.float64)
    ro, rl = attention_fwd(q, k, v, bool(causal), wl, float(scale))
    compare(o, lse, ro, rl, "bf16", label=label, scaled=True)
    got = tuple(_from_bits(tmp_path / f"{n}.bin", x.shape) for n, x in (("dq", q), ("dk", k), ("dv", v)))
    ref, mag = oracle_grads(q, k, v, do, bool(causal), wl, float(scale))
    check_grads(got, ref, mag, "bf16", N, label)
