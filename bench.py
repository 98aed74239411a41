"""Attention-forward benchmark: TFLOP/s and fraction of the MI355X dense
bf16/fp16 matrix-core peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--min-warm-s S] [--workload causal_8k]
                    [--no-cpu-baseline] [--all] [--copy-calibration MiB] [--bwd] [--fp8] [--decode [--splits S]] [--varlen]
                    [--matrix-ceiling]

One step = one forward call (the whole path: Q/K/V tile staging, both
contractions, online softmax, epilogue) over seeded synthetic inputs already
resident in device memory.  Prints ONE JSON line (``--all``: one per
workload, without the CPU baseline).  Besides the rate, the line carries the
mean, median and minimum per-call time from HIP events, the shader clock read
during the timed calls, and -- with the CPU baseline -- the host's CPU model
and BLAS and ``parity``: the timed run's output compared element by element
with the fp64 oracle on every slice the baseline computed.

FLOPs credited per call: 4*d per visible (query, key) pair per head; causal
counts N^2/2 pairs, a window counts the exact visible pairs.

``--fp8`` times the FP8 forward (E4M3 inputs with per-tensor scales, bf16
output) on the headline shape, against the dense fp8 matrix-core peak.

``--decode`` times attention against a key/value cache (few query rows per
sequence, split-KV plus merge) on ``decode_gqa_32k`` (``--all``: every
decoding workload), as algorithmic bytes per second against HBM bandwidth.

``--varlen`` times the packed variable-length forward on
``varlen_causal_16`` (16 sequences of 512-8192 tokens), FLOPs over the exact
visible pairs of every sequence; ``--varlen --bwd`` its backward (one step =
one ``fa.bwd_varlen`` call, credited 2.5 x those FLOPs).

``--matrix-ceiling`` times the vendor bf16 GEMM (torch.matmul, hipBLASLt) on
square 8192^3 and 16384^3 products, once with inputs drawn like the headline
workload's and once with zeros: a reference for how much of the nominal
matrix-core peak the chip sustains under its power limit with such data
(library code, not part of the attention path).

``--bwd`` times the backward instead (one step = one ``fa.bwd`` call: the
row-term prep, dK/dV and dQ kernels) from the forward's o and lse, credited
2.5x the forward's FLOPs (five products of the forward's size).
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

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2, "f32": 157.3}  # dense MFMA (fp32: vector/matrix)
KERNEL_NAME = {"bf16": "fwd_mfma_kernel", "f16": "fwd_mfma_kernel", "f32": "fwd_f32_kernel"}
BWD_KERNELS = "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel"


# sources each forward kernel is compiled from (its launch, host code aside)
FWD_SOURCES = ("fa_fwd_mfma.hip", "fa_mfma_common.h", "fa_internal.h")
FP8_SOURCES = ("fa_fwd_fp8.hip", "fa_mfma_common.h", "fa_internal.h")
F32_SOURCES = ("fa_fwd_f32.hip", "fa_internal.h")


def kernel_source_hash(sources=FWD_SOURCES) -> str:
    """sha256 over a kernel's sources (sorted by name): a stored traffic
    measurement stays valid while these are unchanged."""
    csrc = os.path.join(ROOT, "exact_tiled_attention_04_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(sources):
        h.update(fn.encode())
        h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, sources=FWD_SOURCES):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_info(cores):
    """Host CPU model and the BLAS numpy calls (for the CPU baseline)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "threads": cores}


def parity_fields(errs, tol):
    """Summary of a comparison with the oracle: ``errs`` maps a name to an
    array of absolute errors (or a float); ``tol`` maps the gated names to
    their bounds."""
    import numpy as np
    out = {}
    for name, e in errs.items():
        out[name] = float(np.max(e)) if not np.isscalar(e) else float(e)
    out = {k: (float(f"{v:.3e}") if v else 0.0) for k, v in out.items()}
    out["tol"] = tol
    out["within_tol"] = all(out[k] <= v for k, v in tol.items())
    return out


def cpu_baseline(w, q, k, v, budget_s: float = 12.0, gpu=None):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    every query row of successive (batch, head) slices, as many slices at a
    time as there are host cores (one slice per worker thread, BLAS held to
    one thread each), until ``budget_s`` of wall time has passed.

    With ``gpu = (o, lse)`` (host arrays of the timed run's output), also
    compares every element of the slices the oracle computed with it and
    returns (baseline, parity)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import attention_fwd

    cores = len(os.sched_getaffinity(0))
    flops_per_head = W.metric_flops(w) / (w.B * w.Hq)
    g = w.Hq // w.Hkv
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    done = 0
    eo_max, eo_sum, el_max, n_el, ref_sq = 0.0, 0.0, 0.0, 0, 0.0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while done < len(heads) and time.perf_counter() - t0 < budget_s:
            chunk = heads[done:done + cores]
            qs = np.stack([q[b, h] for b, h in chunk])[None]
            ks = np.stack([k[b, h // g] for b, h in chunk])[None]   # each query head's own K/V head
            vs = np.stack([v[b, h // g] for b, h in chunk])[None]
            ro, rl = attention_fwd(qs, ks, vs, w.causal, w.window_left, w.scale, threads=cores)
            if gpu is not None:
                for i, (b, h) in enumerate(chunk):
                    eo = np.abs(gpu[0][b, h].astype(np.float64) - ro[0, i])
                    eo_max = max(eo_max, float(eo.max()))
                    eo_sum += float(eo.sum())
                    n_el += eo.size
                    ref_sq += float((ro[0, i] ** 2).sum())
                    el_max = max(el_max, float(np.abs(gpu[1][b, h].astype(np.float64) - rl[0, i]).max()))
            done += len(chunk)
    dt = time.perf_counter() - t0
    value = flops_per_head * done / dt / 1e12
    base = {"value": round(value, 6), "unit": "TFLOP/s", "cores": min(cores, len(heads)), "kind": "oracle",
            "sample": f"{done} of {len(heads)} (batch, head) slices, all {w.N} query rows each, "
                      f"fp64 numpy, {dt:.1f} s wall", **host_info(min(cores, len(heads)))}
    if gpu is None:
        return base
    tol = {"o_max_abs": 1e-5} if w.dtype == "f32" else {"o_max_abs": 1e-2, "o_mean_abs": 1e-3, "lse_max_abs": 1e-3}
    par = parity_fields({"o_max_abs": eo_max, "o_mean_abs": eo_sum / max(n_el, 1), "lse_max_abs": el_max}, tol)
    par["o_max_abs_over_rms"] = float(f"{eo_max / max(np.sqrt(ref_sq / max(n_el, 1)), 1e-300):.3e}")
    par["compared"] = f"every element of {done} of {len(heads)} (batch, head) slices against the fp64 oracle"
    return base, par


def calibration_copy(mib: int):
    """A device-to-device copy of ``mib`` MiB (x3), whose counter readings
    calibrate FETCH_SIZE / WRITE_SIZE in the same profiled run."""
    if not mib:
        return None
    import torch
    nbytes = mib * 2 ** 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return f"copied {nbytes} bytes x3 for counter calibration"


def cpu_baseline_bwd(w, q, k, v, do, budget_s: float = 12.0, gpu=None):
    """The fp64 gradient oracle, as it stands, on a bounded sample: whole
    (batch, key/value head) groups, as many at a time as there are host cores
    (BLAS held to one thread each), until ``budget_s`` of wall time has
    passed.  With ``gpu = (dq, dk, dv)`` (host arrays of the timed run's
    output), also compares every element of the groups computed and returns
    (baseline, parity)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import attention_bwd

    cores = len(os.sched_getaffinity(0))
    g = w.Hq // w.Hkv
    flops_per_group = W.bwd_metric_flops(w) / (w.B * w.Hkv)
    groups = [(b, hk) for b in range(w.B) for hk in range(w.Hkv)]
    done = 0
    err = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    mag = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while done < len(groups) and time.perf_counter() - t0 < budget_s:
            chunk = groups[done:done + cores]
            qs = np.concatenate([q[b:b + 1, hk * g:(hk + 1) * g] for b, hk in chunk], axis=1)
            dos = np.concatenate([do[b:b + 1, hk * g:(hk + 1) * g] for b, hk in chunk], axis=1)
            ks = np.concatenate([k[b:b + 1, hk:hk + 1] for b, hk in chunk], axis=1)
            vs = np.concatenate([v[b:b + 1, hk:hk + 1] for b, hk in chunk], axis=1)
            rq, rk, rv = attention_bwd(qs, ks, vs, dos, w.causal, w.window_left, w.scale, threads=cores)
            if gpu is not None:
                for i, (b, hk) in enumerate(chunk):
                    pairs = (("dq", gpu[0][b, hk * g:(hk + 1) * g], rq[0, i * g:(i + 1) * g]),
                             ("dk", gpu[1][b, hk], rk[0, i]), ("dv", gpu[2][b, hk], rv[0, i]))
                    for name, got, ref in pairs:
                        err[name] = max(err[name], float(np.abs(got.astype(np.float64) - ref).max()))
                        mag[name] = max(mag[name], float(np.abs(ref).max()))
            done += len(chunk)
    dt = time.perf_counter() - t0
    base = {"value": round(flops_per_group * done / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(cores, len(groups)), "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, key/value head) groups, all {w.N} rows each, "
                      f"fp64 numpy, {dt:.1f} s wall", **host_info(min(cores, len(groups)))}
    if gpu is None:
        return base
    par = {f"{n}_max_abs": float(f"{err[n]:.3e}") for n in err}
    par.update({f"{n}_max_abs_over_max": float(f"{err[n] / max(mag[n], 1e-300):.3e}") for n in err})
    par["compared"] = (f"every element of {done} of {len(groups)} (batch, key/value head) groups against the fp64 "
                       "gradient oracle; the per-element gate (one rounding of P and dS) is in the GPU tests")
    return base, par


class ClockSampler:
    """Shader-clock and socket-power readings from the driver's metrics table
    (amdsmi ``current_gfxclks``, one value per XCD, and
    ``current_socket_power`` in W; the firmware refreshes them about once per
    second), taken every few milliseconds in a background thread, plus the
    board's power cap.  ``window(t0, t1)`` returns the clock readings taken
    between two ``time.perf_counter()`` instants, ``power_window`` the power
    readings.  Empty when amdsmi is unavailable."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.samples = []
        self.power = []
        self.power_cap_w = None
        self.error = None
        self._stop = threading.Event()
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # no driver access: report no clock
            self.error = repr(e)
            return
        try:
            cap = amdsmi.amdsmi_get_power_cap_info(self._h).get("power_cap")
            if isinstance(cap, (int, float)) and cap > 0:
                self.power_cap_w = cap / 1e6  # reported in microwatts
        except Exception:
            pass
        self._thread = threading.Thread(target=self._run, args=(period_s,), daemon=True)
        self._thread.start()

    def _run(self, period_s):
        while not self._stop.is_set():
            try:
                m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
                if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
                    clks = [m["current_gfxclk"]]
                now = time.perf_counter()
                if clks:
                    self.samples.append((now, sum(clks) / len(clks)))
                pw = m.get("current_socket_power")
                if isinstance(pw, (int, float)) and pw > 0:
                    self.power.append((now, float(pw)))
            except Exception as e:
                self.error = repr(e)
                return
            self._stop.wait(period_s)

    def stop(self):
        self._stop.set()
        if self.error is None:
            self._thread.join()

    def window(self, t0, t1):
        return [c for t, c in self.samples if t0 <= t <= t1]

    def power_window(self, t0, t1):
        return [w for t, w in self.power if t0 <= t <= t1]


def time_steps(step, args, label, stream):
    """W untimed calls, then more untimed calls until at least
    ``args.min_warm_s`` seconds of warm-up have passed (the chip needs ~50
    launches of sustained work to leave its low-clock state, and its clock
    readings refresh about once per second), then K timed calls bracketed by
    device synchronisation, with a HIP event pair recorded on ``stream`` (the
    stream the kernels are launched on) around every call.

    Returns a dict: ``wall`` (seconds for the K calls), ``per_call_ms``,
    ``warmup_extra`` (calls beyond W), ``warm_s``, and ``sclk_mhz`` (clock
    readings taken during the timed calls, or the last one before them) and
    ``power_w`` (socket power during the timed calls and the board's cap, or
    None)."""
    import numpy as np
    import torch
    clock = ClockSampler()
    print(f"[bench] {label}: warmup {args.warmup} (+ until {args.min_warm_s:.2f} s)", file=sys.stderr, flush=True)
    tw = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - tw < args.min_warm_s:
        for _ in range(10):
            step()
        extra += 10
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - tw
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    print(f"[bench] {label}: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clock.stop()
    per_call = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    print(f"[bench] {label}: per-call us " + " ".join(f"{x * 1e3:.1f}" for x in per_call), file=sys.stderr,
          flush=True)
    during = clock.window(t0, t1)
    before = [c for t, c in clock.samples if t < t0]
    sclk = None
    if during or before:
        vals = during if during else before[-1:]
        sclk = {"mean": round(float(np.mean(vals)), 1), "samples": len(vals),
                "when": "during the timed calls" if during else "last reading before the timed calls",
                "source": "amdsmi current_gfxclks, mean over XCDs (refreshed about once per second)"}
    elif clock.error:
        sclk = {"error": clock.error[:200]}
    watts = clock.power_window(t0, t1)
    power = None
    if watts:
        power = {"mean": round(float(np.mean(watts)), 1), "samples": len(watts), "cap": clock.power_cap_w,
                 "source": "amdsmi current_socket_power during the timed calls; cap from amdsmi_get_power_cap_info"}
    return {"wall": t1 - t0, "per_call_ms": per_call, "warmup_extra": extra, "warm_s": warm_s, "sclk_mhz": sclk,
            "power_w": power}


def timing_fields(t, flops_or_bytes, scale=1e12):
    """Per-launch statistics of a ``time_steps`` result: mean, median and
    min in microseconds, and the rate at the mean."""
    import numpy as np
    ms = np.asarray(t["per_call_ms"])
    return {"avg_us": round(float(ms.mean()) * 1e3, 2), "median_us": round(float(np.median(ms)) * 1e3, 2),
            "min_us": round(float(ms.min()) * 1e3, 2),
            "rate_at_avg": flops_or_bytes / (float(ms.mean()) * 1e-3) / scale}


def make_record(args, t, *, metric, work, unit, peak, bound, dtype, config, kernel, traffic=None, per="launch"):
    """The JSON line of one timed workload: ``work`` is the algorithmic FLOPs
    (unit TFLOP/s) or bytes (unit GB/s) of one step; ``value`` is that work
    over the wall time of the K timed steps, ``roofline.achieved`` the same
    work over the mean per-step time from HIP events."""
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    tf = timing_fields(t, work, scale)
    value = work * args.steps / t["wall"] / scale
    return {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_extra": t["warmup_extra"],
        "ms_per_step": round(t["wall"] * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": config,
        "roofline": {"bound": bound, "achieved": round(tf["rate_at_avg"], 3), "peak": peak, "unit": unit,
                     "frac": round(tf["rate_at_avg"] / peak, 4), "traffic": traffic, "kernel": kernel,
                     f"avg_{per}_us": tf["avg_us"], f"median_{per}_us": tf["median_us"],
                     f"min_{per}_us": tf["min_us"]},
        "clock": clock_fields(t, tf, peak, bound),
    }


# The nominal peaks are quoted at the top shader clock; the chip holds a lower
# one under sustained matrix work (power), so the line also prices the
# achieved rate against the peak at the clock read during the timed calls.
NOMINAL_SCLK_MHZ = 2400.0


def clock_fields(t, tf, peak, bound):
    out = {"sclk_mhz": t["sclk_mhz"], "warm_s": round(t["warm_s"], 3)}
    if t.get("power_w"):
        out["power_w"] = t["power_w"]
    s = t["sclk_mhz"]
    mhz = s.get("mean") if isinstance(s, dict) else None
    if bound != "hbm" and mhz:
        out["frac_of_peak_at_measured_clock"] = round(tf["rate_at_avg"] / (peak * mhz / NOMINAL_SCLK_MHZ), 4)
    return out


def run_bwd(args, name, with_cpu):
    import torch

    import exact_tiled_attention_04_amd as fa
    import workloads as W

    w = W.WORKLOADS[name]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    q, k, v = W.make_inputs(w)
    do = W.make_grad(w)
    qd, kd, vd, dod = (torch.from_numpy(x).to(tdt).cuda() for x in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, window_left=w.window_left, scale=w.scale)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(fa._lib.fa_bwd_workspace_size(w.B, w.Hq, w.N) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, window_left=w.window_left, scale=w.scale,
               dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)

    t = time_steps(step, args, f"{name} bwd", stream)
    flops = W.bwd_metric_flops(w)
    config = {"workload": name + " (backward)", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
              "causal": w.causal, "window_left": w.window_left, "scale": w.scale, "seed": w.seed,
              "flops_per_step": flops}
    rec = make_record(args, t, metric="attention bwd TFLOP/s + % of MI355X bf16 MFMA peak (2.5x forward FLOPs)",
                      work=flops, unit="TFLOP/s", peak=PEAK_TFLOPS[w.dtype], bound="mfma", dtype=w.dtype,
                      config=config, kernel=BWD_KERNELS, per="call")
    copy_note = calibration_copy(args.copy_calibration)
    if copy_note:
        rec["calibration"] = copy_note
    if with_cpu:
        print(f"[bench] {name} bwd: cpu baseline (oracle)", file=sys.stderr, flush=True)
        gpu = tuple(x.float().cpu().numpy() for x in (dq, dk, dv))
        rec["cpu_baseline"], rec["parity"] = cpu_baseline_bwd(w, q, k, v, do, gpu=gpu)
    return rec


def run(args, name, with_cpu):
    import torch

    import exact_tiled_attention_04_amd as fa
    import workloads as W

    w = W.WORKLOADS[name]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    q, k, v = W.make_inputs(w)
    qd, kd, vd = (torch.from_numpy(x).to(tdt).cuda() for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fwd(qd, kd, vd, causal=w.causal, window_left=w.window_left, scale=w.scale,
               out=o, lse=lse, stream=stream)

    t = time_steps(step, args, name, stream)
    flops = W.metric_flops(w)
    peak = PEAK_TFLOPS[w.dtype]
    # the headline workload carries the headline metric's name; the others
    # the same measure, named by their config
    unit_name = {"bf16": "bf16 MFMA", "f16": "fp16 MFMA", "f32": "fp32 vector"}[w.dtype]
    metric = f"attention fwd TFLOP/s + % of MI355X {unit_name} peak"
    if name == "causal_8k":
        metric += " (d=128, causal, N=8k)"
    config = {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": w.causal,
              "window_left": w.window_left, "scale": w.scale, "seed": w.seed, "flops_per_step": flops}
    rec = make_record(args, t, metric=metric, work=flops, unit="TFLOP/s", peak=peak,
                      bound="mfma" if w.dtype != "f32" else "alu", dtype=w.dtype, config=config,
                      kernel=KERNEL_NAME[w.dtype],
                      traffic=measured_traffic(name, F32_SOURCES if w.dtype == "f32" else FWD_SOURCES))
    copy_note = calibration_copy(args.copy_calibration)
    if copy_note:
        rec["calibration"] = copy_note
    if with_cpu:
        print(f"[bench] {name}: cpu baseline (oracle) and parity of the timed run's output", file=sys.stderr,
              flush=True)
        gpu = (o.float().cpu().numpy(), lse.cpu().numpy())
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(w, q, k, v, gpu=gpu)
    return rec


def run_fp8(args, name, with_cpu):
    """The FP8 forward on its workload: E4M3 inputs with per-tensor scales
    (the float32 recipe quantised on the host), bf16 output, lse."""
    import torch

    import exact_tiled_attention_04_amd as fa
    import workloads as W

    w = W.FP8_WORKLOADS[name]
    (qb, qs, qf), (kb, ks, kf), (vb, vs, vf) = W.make_fp8_inputs(w)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (qb, kb, vb))
    o = torch.empty(qd.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fwd_fp8(qd, kd, vd, qs, ks, vs, causal=w.causal, window_left=w.window_left, scale=w.scale,
                   out=o, lse=lse, stream=stream)

    t = time_steps(step, args, name, stream)
    flops = W.metric_flops(w)
    config = {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": w.causal,
              "window_left": w.window_left, "scale": w.scale, "seed": w.seed, "scales": [qs, ks, vs],
              "output": "bf16", "flops_per_step": flops}
    rec = make_record(args, t, metric="attention fwd TFLOP/s + % of MI355X fp8 MFMA peak (FP8 E4M3 inputs, d=128, "
                      "causal, N=8k)", work=flops, unit="TFLOP/s", peak=PEAK_TFLOPS["fp8"], bound="mfma",
                      dtype="fp8_e4m3", config=config, kernel="fwd_fp8_kernel",
                      traffic=measured_traffic(name, FP8_SOURCES))
    copy_note = calibration_copy(args.copy_calibration)
    if copy_note:
        rec["calibration"] = copy_note
    if with_cpu:
        print(f"[bench] {name}: cpu baseline (oracle on the dequantised inputs)", file=sys.stderr, flush=True)
        gpu = (o.float().cpu().numpy(), lse.cpu().numpy())
        base, par = cpu_baseline(w, qf, kf, vf, gpu=gpu)
        # FP8 probabilities carry 3 mantissa bits: the per-element gate is
        # the bound of the FP8 tests, not the 16-bit tolerances
        par["tol"] = "per-element bound of the FP8 parity tests (3-bit probabilities)"
        par.pop("within_tol", None)
        rec["cpu_baseline"], rec["parity"] = base, par
    return rec


def cpu_baseline_decode(w, q, k, v, lens, budget_s: float = 12.0, gpu=None):
    """The fp64 cache oracle, as it stands, on a bounded sample: whole
    batches (every head, every row), one worker thread per host core, until
    ``budget_s`` of wall time has passed; reported as GB/s of the same
    algorithmic bytes the GPU line counts.  With ``gpu = (o, lse)``, also
    compares every element of the batches computed and returns (baseline,
    parity)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import attention_fwd_kvcache

    cores = len(os.sched_getaffinity(0))
    done, nbytes = 0, 0
    eo_max, eo_sum, el_max, n_el = 0.0, 0.0, 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while done < w.B and time.perf_counter() - t0 < budget_s:
            b = done
            ro, rl = attention_fwd_kvcache(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], w.causal,
                                           w.window_left, w.scale, threads=cores)
            if gpu is not None:
                eo = np.abs(gpu[0][b:b + 1].astype(np.float64) - ro)
                eo_max, eo_sum, n_el = max(eo_max, float(eo.max())), eo_sum + float(eo.sum()), n_el + eo.size
                fin = np.isfinite(rl)
                assert (np.isfinite(gpu[1][b:b + 1]) == fin).all(), "rows that see no key differ"
                if fin.any():
                    el_max = max(el_max, float(np.abs(gpu[1][b:b + 1][fin] - rl[fin]).max()))
            nbytes += W.decode_bytes(w.replace(B=1), lens[b:b + 1])
            done += 1
    dt = time.perf_counter() - t0
    base = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": min(cores, w.Hq), "kind": "oracle",
            "sample": f"{done} of {w.B} sequences (every head and row), fp64 numpy, {dt:.1f} s wall",
            **host_info(min(cores, w.Hq))}
    if gpu is None:
        return base
    par = parity_fields({"o_max_abs": eo_max, "o_mean_abs": eo_sum / max(n_el, 1), "lse_max_abs": el_max},
                        {"o_max_abs": 1e-2, "o_mean_abs": 1e-3, "lse_max_abs": 1e-3})
    par["compared"] = f"every element of {done} of {w.B} sequences against the fp64 cache oracle"
    return base, par


def run_decode(args, name, with_cpu):
    """Attention against a key/value cache: one step = one fa.fwd_kvcache(_paged)
    call (the split kernel and, with more than one split, the merge), cache
    resident in device memory.  Metric: algorithmic bytes per second."""
    import numpy as np
    import torch

    import exact_tiled_attention_04_amd as fa
    import workloads as W

    w = W.DECODE_WORKLOADS[name]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    q, k, v, lens = W.make_decode_inputs(w)
    qd = torch.from_numpy(q).to(tdt).cuda()
    sd = torch.from_numpy(lens).cuda()
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if w.page_size:
        kp, vp, table = W.build_pages(k, v, lens, w.page_size, w.seed)
        kd, vd = (torch.from_numpy(x).to(tdt).cuda() for x in (kp, vp))
        td = torch.from_numpy(table).cuda()
        nk = w.page_size * table.shape[1]
    else:
        kd, vd = (torch.from_numpy(x).to(tdt).cuda() for x in (k, v))
        nk = w.Nk
    # the caller knows its cache lengths: let the library pick splits for them
    splits = args.splits if args.splits else fa.kvcache_num_splits(lens, w.Hq, w.Hkv, w.Nq, nk, w.causal,
                                                                   w.window_left)
    ws_bytes = fa._lib.fa_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, nk, w.d, splits)
    ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device="cuda")

    if w.page_size:
        def step():
            fa.fwd_kvcache_paged(qd, kd, vd, td, sd, causal=w.causal, window_left=w.window_left, scale=w.scale,
                                 num_splits=splits, out=o, lse=lse, workspace=ws, stream=stream)
    else:
        def step():
            fa.fwd_kvcache(qd, kd, vd, sd, causal=w.causal, window_left=w.window_left, scale=w.scale,
                           num_splits=splits, out=o, lse=lse, workspace=ws, stream=stream)

    t = time_steps(step, args, name, stream)
    nbytes = W.decode_bytes(w, lens)
    config = {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
              "causal": w.causal, "window_left": w.window_left, "page_size": w.page_size, "lengths": w.lengths,
              "total_keys": int(np.sum(lens)), "seed": w.seed, "splits": splits, "bytes_per_step": nbytes}
    rec = make_record(args, t, metric="attention decode GB/s + % of MI355X HBM bandwidth (8 TB/s)", work=nbytes,
                      unit="GB/s", peak=8000.0, bound="hbm", dtype=w.dtype, config=config,
                      kernel="decode_split_kernel" + (" + decode_merge_kernel" if splits > 1 else ""), per="call")
    copy_note = calibration_copy(args.copy_calibration)
    if copy_note:
        rec["calibration"] = copy_note
    if with_cpu:
        print(f"[bench] {name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        gpu = (o.float().cpu().numpy(), lse.cpu().numpy())
        rec["cpu_baseline"], rec["parity"] = cpu_baseline_decode(w, q, k, v, lens, gpu=gpu)
    return rec


def cpu_baseline_varlen(w, q, k, v, cu, budget_s: float = 12.0, gpu=None):
    """The fp64 packed oracle, as it stands, on a bounded sample: whole
    sequences from the first, with every head and row, until ``budget_s`` of
    wall time has passed (BLAS on one thread per worker).  With ``gpu = (o,
    lse)`` (o [total][Hq][d], lse [Hq][total]), also compares every element
    of the sequences computed and returns (baseline, parity)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import attention_fwd_varlen

    cores = len(os.sched_getaffinity(0))
    done, flops = 0, 0.0
    eo_max, eo_sum, el_max, n_el = 0.0, 0.0, 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while done < w.B and time.perf_counter() - t0 < budget_s:
            a, z = int(cu[done]), int(cu[done + 1])
            sub = np.array([0, z - a], dtype=np.int32)
            ro, rl = attention_fwd_varlen(q[a:z], k[a:z], v[a:z], sub, sub, w.causal, w.window_left, w.scale,
                                          threads=cores)
            if gpu is not None:
                eo = np.abs(gpu[0][a:z].astype(np.float64) - ro)
                eo_max, eo_sum, n_el = max(eo_max, float(eo.max())), eo_sum + float(eo.sum()), n_el + eo.size
                el_max = max(el_max, float(np.abs(gpu[1][:, a:z].astype(np.float64) - rl).max()))
            flops += W.varlen_metric_flops(w, sub)
            done += 1
    dt = time.perf_counter() - t0
    base = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": min(cores, w.Hq), "kind": "oracle",
            "sample": f"{done} of {w.B} sequences (every head and row), fp64 numpy, {dt:.1f} s wall",
            **host_info(min(cores, w.Hq))}
    if gpu is None:
        return base
    par = parity_fields({"o_max_abs": eo_max, "o_mean_abs": eo_sum / max(n_el, 1), "lse_max_abs": el_max},
                        {"o_max_abs": 1e-2, "o_mean_abs": 1e-3, "lse_max_abs": 1e-3})
    par["compared"] = f"every element of {done} of {w.B} sequences against the fp64 packed oracle"
    return base, par


def run_varlen(args, name, with_cpu):
    """Packed sequences of different lengths: one step = one fa.fwd_varlen call."""
    import numpy as np
    import torch

    import exact_tiled_attention_04_amd as fa
    import workloads as W

    w = W.VARLEN_WORKLOADS[name]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    q, k, v, cu = W.make_varlen_inputs(w)
    qd, kd, vd = (torch.from_numpy(x).to(tdt).cuda() for x in (q, k, v))
    cud = torch.from_numpy(cu).cuda()
    maxlen = int(np.diff(cu).max())
    o = torch.empty_like(qd)
    lse = torch.empty((w.Hq, q.shape[0]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fwd_varlen(qd, kd, vd, cud, cud, maxlen, maxlen, causal=w.causal, window_left=w.window_left,
                      scale=w.scale, out=o, lse=lse, stream=stream)

    t = time_steps(step, args, name, stream)
    flops = W.varlen_metric_flops(w, cu)
    config = {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "lengths": [int(x) for x in np.diff(cu)],
              "total_tokens": int(cu[-1]), "d": w.d, "causal": w.causal, "window_left": w.window_left,
              "scale": w.scale, "seed": w.seed, "flops_per_step": flops}
    rec = make_record(args, t, metric="attention fwd TFLOP/s + % of MI355X bf16 MFMA peak (packed sequences of "
                      "different lengths)", work=flops, unit="TFLOP/s", peak=PEAK_TFLOPS[w.dtype], bound="mfma",
                      dtype=w.dtype, config=config, kernel="fwd_mfma_kernel (packed)")
    if with_cpu:
        print(f"[bench] {name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        gpu = (o.float().cpu().numpy(), lse.cpu().numpy())
        rec["cpu_baseline"], rec["parity"] = cpu_baseline_varlen(w, q, k, v, cu, gpu=gpu)
    return rec


def run_varlen_bwd(args, name, with_cpu):
    """Packed sequences of different lengths, backward: one step = one
    fa.bwd_varlen call (dq, dk, dv from the forward's o and lse, which are
    computed once before the timed region).  Credited work is 2.5 times the
    forward's metric FLOPs (the five products of the backward against the
    forward's two), the convention of the batched backward line."""
    import numpy as np
    import torch

    import exact_tiled_attention_04_amd as fa
    import workloads as W

    w = W.VARLEN_WORKLOADS[name]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    q, k, v, cu = W.make_varlen_inputs(w)
    do = W.random_grad(w.seed + 100, w.dtype, 1, w.Hq, q.shape[0], w.d)[0].transpose(1, 0, 2)
    qd, kd, vd = (torch.from_numpy(x).to(tdt).cuda() for x in (q, k, v))
    dod = torch.from_numpy(np.ascontiguousarray(do)).to(tdt).cuda()
    cud = torch.from_numpy(cu).cuda()
    maxlen = int(np.diff(cu).max())
    o, lse = fa.fwd_varlen(qd, kd, vd, cud, cud, maxlen, maxlen, causal=w.causal, window_left=w.window_left,
                           scale=w.scale)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(max(1, fa._lib.fa_bwd_workspace_size(1, w.Hq, q.shape[0]) // 4), dtype=torch.float32,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.bwd_varlen(qd, kd, vd, o, lse, dod, cud, cud, maxlen, maxlen, causal=w.causal,
                      window_left=w.window_left, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)

    t = time_steps(step, args, name, stream)
    flops = 2.5 * W.varlen_metric_flops(w, cu)
    config = {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "lengths": [int(x) for x in np.diff(cu)],
              "total_tokens": int(cu[-1]), "d": w.d, "causal": w.causal, "window_left": w.window_left,
              "scale": w.scale, "seed": w.seed, "flops_per_step": flops}
    rec = make_record(args, t, metric="attention bwd TFLOP/s + % of MI355X bf16 MFMA peak (packed sequences of "
                      "different lengths)", work=flops, unit="TFLOP/s", peak=PEAK_TFLOPS[w.dtype], bound="mfma",
                      dtype=w.dtype, config=config, kernel="bwd_prep + bwd_dkdv + bwd_dq (packed)", per="call")
    if with_cpu:
        print(f"[bench] {name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_varlen_bwd(w, q, k, v, do, cu)
    return rec


def cpu_baseline_varlen_bwd(w, q, k, v, do, cu, budget_s: float = 12.0):
    """The fp64 packed gradient oracle, as it stands, on a bounded sample:
    whole sequences from the first until ``budget_s`` of wall time has
    passed; credited like the GPU line (2.5 x the forward's FLOPs)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import attention_bwd_varlen

    cores = len(os.sched_getaffinity(0))
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while done < w.B and time.perf_counter() - t0 < budget_s:
            a, z = int(cu[done]), int(cu[done + 1])
            sub = np.array([0, z - a], dtype=np.int32)
            attention_bwd_varlen(q[a:z], k[a:z], v[a:z], do[a:z], sub, sub, w.causal, w.window_left, w.scale,
                                 threads=cores)
            flops += 2.5 * W.varlen_metric_flops(w, sub)
            done += 1
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": min(cores, w.Hkv), "kind": "oracle",
            "sample": f"{done} of {w.B} sequences (every head and row), fp64 numpy, {dt:.1f} s wall",
            **host_info(min(cores, w.Hkv))}


def run_matrix_ceiling(args):
    """bf16 GEMM throughput of the vendor library on inputs like the headline
    workload's (0.5 * N(0, 1), rounded to bf16) and on zeros, one JSON line
    per case: the matrix cores' sustained rate under the power limit depends
    on the data's bit activity, which sets the clock."""
    import torch
    recs = []
    for M in (8192, 16384):
        g = torch.Generator(device="cuda")
        g.manual_seed(2)
        a = (torch.randn(M, M, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        b = (torch.randn(M, M, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        for data in ("0.5*N(0,1)", "zeros"):
            if data == "zeros":
                a.zero_()
                b.zero_()
            steps = max(5, args.steps // (10 if M == 8192 else 40))
            warm = max(5, args.warmup // (10 if M == 8192 else 40))
            sub = argparse.Namespace(steps=steps, warmup=warm, min_warm_s=args.min_warm_s)
            stream = torch.cuda.current_stream()
            per_call = time_steps(lambda: torch.matmul(a, b), sub, f"gemm {M} {data}", stream)["per_call_ms"]
            ms = sorted(per_call)[len(per_call) // 2]
            tf = 2.0 * M ** 3 / (ms * 1e-3) / 1e12
            recs.append({"metric": "bf16 GEMM TFLOP/s (torch.matmul / hipBLASLt), reference ceiling",
                         "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warm,
                         "ms_per_step": round(ms, 4), "higher_is_better": True,
                         "pct_of_peak": round(100 * tf / PEAK_TFLOPS["bf16"], 1), "dtype": "bf16",
                         "data": data, "config": {"workload": f"gemm_{M}", "M": M, "N": M, "K": M}})
    return recs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU needs ~30 ms of sustained work to leave its low-clock state
    # (per-launch time settles after ~50 launches of the causal 8k workload,
    # then drifts by ~1% over seconds as the chip warms): whatever --warmup
    # asks for, untimed calls continue for --min-warm-s seconds, so the timed
    # steps measure the steady state and the clock reading taken during them
    # (refreshed about once per second) describes that state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warm-s", type=float, default=1.0,
                    help="keep warming up (untimed calls, reported as warmup_extra) until this many seconds "
                         "have passed, whatever --warmup is")
    ap.add_argument("--workload", default="causal_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="one line per workload (no CPU baseline)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="also run a device copy of this size (counter calibration)")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass instead of the forward")
    ap.add_argument("--fp8", action="store_true", help="time the FP8 forward (workload causal_8k_fp8)")
    ap.add_argument("--decode", action="store_true",
                    help="time attention against a key/value cache (workload decode_gqa_32k, or --workload)")
    ap.add_argument("--splits", type=int, default=None, help="--decode: split count (default: the library's)")
    ap.add_argument("--varlen", action="store_true",
                    help="time the packed variable-length forward (workload varlen_causal_16; with --bwd its "
                         "backward)")
    ap.add_argument("--matrix-ceiling", action="store_true",
                    help="time the vendor bf16 GEMM on headline-like data and on zeros (reference)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward kernel runs on a single device "
              "(multi-GPU sharding of batch x heads needs no communication and is not launched here).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import workloads as W
    if args.matrix_ceiling:
        for rec in run_matrix_ceiling(args):
            print(json.dumps(rec), flush=True)
        return
    if args.varlen:
        name = args.workload if args.workload in W.VARLEN_WORKLOADS else "varlen_causal_16"
        runner = run_varlen_bwd if args.bwd else run_varlen
        print(json.dumps(runner(args, name, not args.no_cpu_baseline)), flush=True)
        return
    if args.decode:
        names = sorted(W.DECODE_WORKLOADS) if args.all else \
            [args.workload if args.workload in W.DECODE_WORKLOADS else W.DECODE_HEADLINE]
        for name in names:
            print(json.dumps(run_decode(args, name, not args.all and not args.no_cpu_baseline)), flush=True)
        return
    if args.fp8:
        name = args.workload if args.workload in W.FP8_WORKLOADS else "causal_8k_fp8"
        print(json.dumps(run_fp8(args, name, not args.no_cpu_baseline)), flush=True)
        return
    if args.bwd:
        names = [n for n in W.ORDER if W.WORKLOADS[n].dtype != "f32"] if args.all else [args.workload]
        for name in names:
            print(json.dumps(run_bwd(args, name, not args.all and not args.no_cpu_baseline)), flush=True)
        return
    if args.all:
        for name in W.ORDER:
            print(json.dumps(run(args, name, False)), flush=True)
        return
    print(json.dumps(run(args, args.workload, not args.no_cpu_baseline)), flush=True)


if __name__ == "__main__":
    main()
