"""Helpers for GPU tests: upload seeded inputs, run the HIP path through the
C ABI, compare with the oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import exact_tiled_attention_04_amd as fa

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Tolerances on O (max abs, mean abs) and on lse (max abs), per input type.
TOL = {
    "f32": dict(o_max=1e-5, o_mean=1e-5, lse=1e-5),
    "f16": dict(o_max=1e-2, o_mean=1e-3, lse=1e-3),
    "bf16": dict(o_max=1e-2, o_mean=1e-3, lse=1e-3),
}


def announce(msg: str) -> None:
    """Name the case before a GPU step, so a run that dies says where."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPE[dtype]).cuda()


def run_gpu(q, k, v, dtype, causal=False, window_left=-1, scale=None, label=""):
    """Upload float32 arrays (exact in dtype), run, return (o, lse) as fp64 numpy."""
    announce(f"{label} dtype={dtype} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} wl={window_left}")
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window_left=window_left, scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def compare(o, lse, o_ref, lse_ref, dtype, label="", scaled=False):
    """Check (o, lse) against the oracle.

    scaled=False: the flat bounds of TOL (used for the five workloads).
    scaled=True: for 16-bit types the O bounds grow with the output's size,
    max |dO_i| <= 1e-2 * max(1, |O_ref,i|) and mean |dO| <= 1e-3 * max(1,
    mean |O_ref|); below magnitude 1 these are the flat bounds.  A 16-bit
    output of magnitude m is itself rounded by up to 2^-9 m (bf16), which
    exceeds a flat 1e-2 once m >= 4; edge shapes with very few visible keys
    produce such outputs.
    """
    tol = TOL[dtype]
    err = np.abs(o - o_ref)
    if scaled and dtype != "f32" and err.size:
        err = err / np.maximum(1.0, np.abs(o_ref))
    lerr = np.abs(lse - lse_ref)
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    max_e, mean_e, lmax = float(err.max(initial=0)), float(err.mean()) if err.size else 0.0, float(lerr.max(initial=0))
    rms = float(np.sqrt(np.mean(o_ref ** 2))) if o_ref.size else 1.0
    print(f"[parity] {label} dtype={dtype} o_max={max_e:.3e} o_mean={mean_e:.3e} lse_max={lmax:.3e} "
          f"o_max/rms={max_e / max(rms, 1e-30):.3e}", file=sys.stderr, flush=True)
    assert max_e <= tol["o_max"], f"{label}: max |dO| {max_e} > {tol['o_max']}"
    assert mean_e <= tol["o_mean"], f"{label}: mean |dO| {mean_e} > {tol['o_mean']}"
    assert lmax <= tol["lse"], f"{label}: max |dlse| {lmax} > {tol['lse']}"
    return max_e, mean_e, lmax


# unit roundoff of the probabilities fed to the P V product (the 16-bit
# kernels round P to the input type; the fp32 kernel keeps it in fp32) and
# of the stored output
UNIT_P = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 0.0}
UNIT_OUT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
SUBNORMAL_ABS = {"bf16": 0.0, "f16": 2.0 ** -25, "f32": 0.0}


def check_rounding_bound(o, lse, q, k, v, causal, wl, scale, dtype, label=""):
    """Every element of (o, lse) under a bound derived from the forward
    kernels' arithmetic, against the fp64 oracle's magnitudes:

        |dO| <= (u_P + (N + 8) 2^-24 + 2^-20 + 2 d 2^-24 S) P|V| + u_out |O|
                + s (N max|V| + 1) + 2^-100 max|O|
        |dlse| <= d 2^-24 S + (N + 8) 2^-24 + 2^-20 (16 + |lse|)

    u_P: rounding of P before the P V product; N 2^-24: fp32 accumulation
    over up to N keys; 2^-20: the exp2 and scale approximations; S = max
    over visible keys of |scale| sum_c |q_c k_c| (``sabs``), so d 2^-24 S
    bounds each score's fp32 error and 2 d 2^-24 S the relative change of a
    probability it causes; u_out: rounding of the stored output; s: the
    absolute rounding error of a probability below the type's normal range
    (fp16: 2^-25; the kernels round unnormalised probabilities whose row
    maximum is at least 1, so after the division by the row sum it stays at
    most s per key) and of a stored output below that range.  The floor
    covers probabilities below fp32's range."""
    from oracle import attention_fwd
    ro, rl, mag = attention_fwd(q, k, v, causal, wl, scale, tail=0.0)
    N, d = k.shape[2], q.shape[3]
    s = mag["sabs"][..., None]
    bound = ((UNIT_P[dtype] + (N + 8) * 2.0 ** -24 + 2.0 ** -20 + 2 * d * 2.0 ** -24 * s) * mag["pv"]
             + UNIT_OUT[dtype] * np.abs(ro) + SUBNORMAL_ABS[dtype] * (N * float(np.abs(v).max(initial=0)) + 1.0)
             + 2.0 ** -100 * float(np.abs(ro).max(initial=0)))
    lbound = d * 2.0 ** -24 * mag["sabs"] + (N + 8) * 2.0 ** -24 + 2.0 ** -20 * (16 + np.abs(rl))
    err, lerr = np.abs(o - ro), np.abs(lse - rl)
    worst = float((err / np.maximum(bound, 1e-300)).max(initial=0))
    lworst = float((lerr / lbound).max(initial=0))
    print(f"[bound] {label} dtype={dtype} worst err/bound O {worst:.3f} lse {lworst:.3f}", file=sys.stderr, flush=True)
    assert (err <= bound).all(), f"{label}: O exceeds the rounding bound (worst ratio {worst:.3f})"
    assert (lerr <= lbound).all(), f"{label}: lse exceeds the rounding bound (worst ratio {lworst:.3f})"


def sample_rows(N: int, rng: np.random.Generator, n_random: int = 48, block: int = 128):
    """First and last rows, rows around query-block and key-tile edges, random rows."""
    rows = {0, 1, N - 1, N - 2}
    for e in range(0, N, block * max(1, N // (block * 8))):
        for d in (-1, 0, 31, 32, 63, 64):
            if 0 <= e + d < N:
                rows.add(e + d)
    rows.update(rng.integers(0, N, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)
