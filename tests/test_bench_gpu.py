"""The benchmark's JSON line, end to end on the GPU: each mode runs a few
calls in a subprocess and must print one line that carries the fields the
measurement contract names (small workloads, so the whole test takes
seconds)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

COMMON = ["--steps", "3", "--warmup", "1", "--min-warm-s", "0"]


def _run(*args):
    print(f"[bench] {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, "bench.py", *args, *COMMON], cwd=ROOT, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip().startswith("{")]
    assert len(lines) >= 1, r.stdout[-2000:]
    return [json.loads(ln) for ln in lines]


def _check_line(rec, unit, bound):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "warmup_extra", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "clock"):
        assert key in rec, key
    assert rec["unit"] == unit and rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["higher_is_better"] is True
    assert rec["data"] == "synthetic" and "workload" in rec["config"]
    roof = rec["roofline"]
    assert roof["bound"] == bound and 0 < roof["frac"] < 1.5 and roof["achieved"] > 0 and roof["peak"] > 0


def test_forward_line_with_cpu_baseline_and_parity():
    (rec,) = _run("--workload", "bf16_n1k_d64")
    _check_line(rec, "TFLOP/s", "mfma")
    base = rec["cpu_baseline"]
    assert base["kind"] == "oracle" and base["value"] > 0 and base["cores"] >= 1 and base["sample"]
    assert rec["parity"]["within_tol"] is True


def test_backward_decode_fp8_and_packed_lines():
    (rec,) = _run("--bwd", "--workload", "bf16_n1k_d64", "--no-cpu-baseline")
    _check_line(rec, "TFLOP/s", "mfma")
    (rec,) = _run("--decode", "--no-cpu-baseline")
    _check_line(rec, "GB/s", "hbm")
    (rec,) = _run("--fp8", "--no-cpu-baseline")
    _check_line(rec, "TFLOP/s", "mfma")
    (rec,) = _run("--varlen", "--no-cpu-baseline")
    _check_line(rec, "TFLOP/s", "mfma")
