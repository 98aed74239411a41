"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 gradient
oracle, through the C ABI (``fa.bwd`` -> ``fa_bwd``).

Inputs: the seeded workload recipe (q, k, v) and its upstream gradient recipe
(dO); o and lse come from this library's own forward, as a caller would pass
them.  The oracle differentiates the exact forward.

Bound (derived from the arithmetic of the kernels): the kernels round P (for
dV) and dS (for dQ, dK) once to the input type, unit roundoff u (bf16 2^-8,
fp16 2^-11), form D_i from the rounded forward output, and accumulate in fp32
over up to n terms (n = N keys for dQ; n = G N query rows for dK and dV,
whose key/value head is shared by the G query heads of its group).  Per
element,

    |got - ref| <= (2u + n 2^-24 + e_P) (M + M_f) + s (M_v + 1) + u |ref| + 2^-100 max|ref|

with M the same product over absolute values (|P|^T|dO|, |scale| |dS||K|,
|scale| |dS|^T|Q|), M_f the row-term product (zero for dV) and M_v the
product with the visibility matrix in place of P or dS (Vis^T|dO|,
|scale| Vis|K|, |scale| Vis^T|Q|); all three come from the oracle.  s is the
absolute rounding error of a value below the type's normal range (an entry
of P or dS, or the stored gradient): fp16's subnormals (below 2^-14) are
spaced 2^-24, so s = 2^-25 for fp16, while
bfloat16 has fp32's exponent range (s = 0; the floor below covers it).
e_P = 2 d 2^-24 S + (N + 8) 2^-24 + 2^-20 (17 + S + ln(N + 1)) is the
relative error of the rebuilt P = exp(scale s - lse): the fp32 score of the
backward and of the forward (d 2^-24 S each, S = |scale| max||q|| max||k||
bounding every |scale| sum_c |q_c k_c|), the forward's fp32 row sum and
the exp2, log and scale approximations.  The last term is an absolute floor for probabilities that
underflow fp32 (scores more than ~87 units below their row's maximum), far
below any visible contribution.  Mean errors are also reported.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from oracle import attention_bwd
from tests.gpu_util import announce, to_dev
from workloads import WORKLOADS, make_grad, make_inputs, random_grad, random_inputs

pytestmark = pytest.mark.gpu

UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
# largest absolute rounding error of a value below the type's normal range
# (fp16 subnormals are spaced 2^-24; bf16 shares fp32's exponent range, where
# the floor below covers it)
SUBNORMAL_ABS = {"bf16": 0.0, "f16": 2.0 ** -25}


def run_bwd_gpu(q, k, v, do, dtype, causal, wl, scale, label=""):
    announce(f"bwd {label} dtype={dtype} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} wl={wl}")
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window_left=wl, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, window_left=wl, scale=scale)
    torch.cuda.synchronize()
    return tuple(x.double().cpu().numpy() for x in (dq, dk, dv))


def check_grads(got, ref, mag, dtype, N, label=""):
    """Every element of (dq, dk, dv) under the bound of the module doc.  N is
    the longest sequence: dQ accumulates over up to N keys, dK and dV of a
    key/value head over up to G * N query rows (the group's G query heads
    share it), so the fp32 accumulation term counts those."""
    u = UNIT[dtype]
    G = got[0].shape[1] // got[1].shape[1]   # heads sit on axis 1 in both layouts
    terms = {"dq": N, "dk": G * N, "dv": G * N}
    # relative error of the rebuilt probabilities: the backward's fp32 score
    # and the forward's logsumexp (its score error, sum and log) enter
    # exp(scale s - lse)
    S, d = mag["score_size"], got[0].shape[-1]
    e_p = 2 * d * 2.0 ** -24 * S + (N + 8) * 2.0 ** -24 + 2.0 ** -20 * (17 + S + np.log(N + 1))
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        gamma = terms[name] * 2.0 ** -24
        assert np.isfinite(g).all(), f"{label}: non-finite {name}"
        m = mag[name] + (mag[name + "_f"] if name + "_f" in mag else 0.0)
        # fp32 flushes probabilities below its range (scores ~100 units below
        # the row max): allow an absolute floor far below any visible value
        floor = 2.0 ** -100 * float(np.abs(r).max(initial=0))
        # a P or dS entry below the normal range is rounded with an absolute
        # error: summed over the visible pairs (the oracle's visibility products)
        sub = SUBNORMAL_ABS[dtype] * (mag[name + "_v"] + 1.0)   # ... and the stored gradient itself
        bound = (2 * u + gamma + e_p) * m + sub + u * np.abs(r) + floor
        err = np.abs(g - r)
        worst = float((err / np.maximum(bound, 1e-300)).max(initial=0))
        rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
        mean_rel = float(err.mean() / max(np.abs(r).mean(), 1e-300)) if r.size else 0.0
        print(f"[parity-bwd] {label} {name} dtype={dtype} max_err={err.max(initial=0):.3e} rms_ref={rms:.3e} "
              f"mean_err/mean_ref={mean_rel:.3e} worst err/bound={worst:.3f}", file=sys.stderr, flush=True)
        assert (err <= bound).all(), f"{label}: {name} exceeds the bound (worst ratio {worst:.3f})"


def score_size(q, k, scale):
    """|scale| max_i ||q_i|| max_j ||k_j||: by Cauchy-Schwarz at least
    |scale| sum_c |q_ic| |k_jc| for every (query, key) pair, i.e. a bound on
    every score's size and on what its fp32 sum accumulates."""
    nq = float(np.sqrt((np.asarray(q, np.float64) ** 2).sum(axis=-1)).max(initial=0.0))
    nk = float(np.sqrt((np.asarray(k, np.float64) ** 2).sum(axis=-1)).max(initial=0.0))
    return abs(scale) * nq * nk


def oracle_grads(q, k, v, do, causal, wl, scale):
    dq, dk, dv, mag = attention_bwd(q, k, v, do, causal, wl, scale, bounds=True)
    mag["score_size"] = score_size(q, k, scale)
    return (dq, dk, dv), mag


# --- edge shapes: ragged lengths, one to several tiles, every mask, GQA ------

EDGE_N = [1, 33, 64, 100, 129, 300]
EDGE_MASKS = [(False, -1), (True, -1), (True, 0), (True, 50), (False, 40)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", EDGE_N)
def test_bwd_edge_shapes(dtype, d, N):
    B, Hq, Hkv = 2, 4, 2
    q, k, v = random_inputs(900 + N + d, dtype, B, Hq, Hkv, N, d)
    do = random_grad(950 + N + d, dtype, B, Hq, N, d)
    scale = d ** -0.5
    for causal, wl in EDGE_MASKS:
        label = f"edge N={N} d={d} causal={causal} wl={wl}"
        got = run_bwd_gpu(q, k, v, do, dtype, causal, wl, scale, label)
        ref, mag = oracle_grads(q, k, v, do, causal, wl, scale)
        check_grads(got, ref, mag, dtype, N, label)


@pytest.mark.parametrize("G", [1, 3, 8])
def test_bwd_gqa_groups(G):
    """dK and dV of a shared head sum over its whole query-head group."""
    B, Hkv, N, d = 1, 2, 200, 128
    q, k, v = random_inputs(960 + G, "bf16", B, Hkv * G, Hkv, N, d)
    do = random_grad(970 + G, "bf16", B, Hkv * G, N, d)
    for causal, wl in [(True, -1), (False, 70)]:
        label = f"gqa G={G} causal={causal} wl={wl}"
        got = run_bwd_gpu(q, k, v, do, "bf16", causal, wl, 0.09, label)
        ref, mag = oracle_grads(q, k, v, do, causal, wl, 0.09)
        check_grads(got, ref, mag, "bf16", N, label)


@pytest.mark.parametrize("mult", [4.0, 12.0])
def test_bwd_large_scores(mult):
    """Peaked softmax rows (scores spread over tens of units)."""
    q, k, v = random_inputs(980, "bf16", 1, 2, 1, 256, 64, mult=mult)
    do = random_grad(981, "bf16", 1, 2, 256, 64)
    for causal in (False, True):
        label = f"large mult={mult} causal={causal}"
        got = run_bwd_gpu(q, k, v, do, "bf16", causal, -1, 0.125, label)
        ref, mag = oracle_grads(q, k, v, do, causal, -1, 0.125)
        check_grads(got, ref, mag, "bf16", 256, label)


# --- the five workloads' backward at reduced sizes (same recipe) -------------

REDUCED = {
    "bf16_n1k_d64": dict(B=1, Hq=4, Hkv=4),
    "causal_8k": dict(B=1, Hq=2, Hkv=2, N=1024),
    "gqa_f16_4k": dict(B=1, Hq=8, Hkv=2, N=1024),
    "swa_32k": dict(B=1, Hq=2, Hkv=2, N=2048),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_bwd_workloads_reduced(name):
    w = WORKLOADS[name]
    over = REDUCED[name]
    wl = w.window_left if name != "swa_32k" else 256
    q, k, v = make_inputs(w, **over)
    do = make_grad(w, **{x: over[x] for x in ("B", "Hq", "N") if x in over})
    N = q.shape[2]
    got = run_bwd_gpu(q, k, v, do, w.dtype, w.causal, wl, w.scale, f"{name} reduced")
    ref, mag = oracle_grads(q, k, v, do, w.causal, wl, w.scale)
    check_grads(got, ref, mag, w.dtype, N, f"{name} reduced")


# --- full sizes: every element, in the benchmark's launch shape -------------

@pytest.mark.parametrize("name", ["causal_8k", "gqa_f16_4k"])
def test_bwd_full_size_every_element(name):
    """The whole problem at full size on the GPU; the oracle checks every
    element of dq, dk and dv (its worker threads each hold BLAS to one
    thread)."""
    from threadpoolctl import threadpool_limits
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    do = make_grad(w)
    got = run_bwd_gpu(q, k, v, do, w.dtype, w.causal, w.window_left, w.scale, f"{name} full")
    with threadpool_limits(limits=1):
        ref, mag = oracle_grads(q, k, v, do, w.causal, w.window_left, w.scale)
    check_grads(got, ref, mag, w.dtype, w.N, f"{name} full, every element")


# --- properties -------------------------------------------------------------

def test_bwd_is_deterministic():
    q, k, v = random_inputs(990, "bf16", 2, 8, 2, 700, 128)
    do = random_grad(991, "bf16", 2, 8, 700, 128)
    a = run_bwd_gpu(q, k, v, do, "bf16", True, 300, 0.1, "determinism 1")
    b = run_bwd_gpu(q, k, v, do, "bf16", True, 300, 0.1, "determinism 2")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bwd_zero_upstream_gives_zero_gradients():
    q, k, v = random_inputs(992, "f16", 1, 2, 1, 150, 64)
    do = np.zeros((1, 2, 150, 64), dtype=np.float32)
    for x in run_bwd_gpu(q, k, v, do, "f16", True, -1, 0.125, "zero dO"):
        assert (x == 0).all()


def test_bwd_rejects_f32_and_bad_shapes():
    q = torch.zeros(1, 2, 64, 64, device="cuda")
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 2, 64, device="cuda")
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, o, lse, o)
    qb = q.to(torch.bfloat16)
    with pytest.raises(ValueError):
        fa.bwd(qb, qb, qb, qb, lse[:, :1], qb)
    with pytest.raises(fa.FaError):
        fa.bwd(qb[..., :48].contiguous(), qb[..., :48].contiguous(), qb[..., :48].contiguous(),
               qb[..., :48].contiguous(), lse, qb[..., :48].contiguous())


def test_bwd_side_stream_and_caller_buffers():
    """Caller-provided outputs and workspace on a side stream give the same
    bits as the default path."""
    q, k, v = random_inputs(993, "bf16", 1, 4, 2, 257, 128)
    do = random_grad(994, "bf16", 1, 4, 257, 128)
    ref = run_bwd_gpu(q, k, v, do, "bf16", True, -1, 0.1, "side stream reference")
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=True, scale=0.1)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(fa._lib.fa_bwd_workspace_size(1, 4, 257) // 4, dtype=torch.float32, device="cuda")
    announce("bwd side stream")
    with torch.cuda.stream(s):
        fa.bwd(qd, kd, vd, o, lse, dod, causal=True, scale=0.1, dq=dq, dk=dk, dv=dv, workspace=ws, stream=s)
    s.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        np.testing.assert_array_equal(x.double().cpu().numpy(), y)


def test_differentiable_attention_matches_fwd_and_bwd():
    """fa.attend under torch autograd gives the same bits as calling fwd
    and bwd directly, and its gradients are within the oracle's bound."""
    q, k, v = random_inputs(995, "bf16", 1, 4, 2, 200, 128)
    do = random_grad(996, "bf16", 1, 4, 200, 128)
    ref = run_bwd_gpu(q, k, v, do, "bf16", True, 60, 0.1, "autograd reference")
    qd, kd, vd, dod = (to_dev(x, "bf16").requires_grad_(i < 3) for i, x in enumerate((q, k, v, do)))
    announce("autograd attention")
    o = fa.attend(qd, kd, vd, causal=True, window_left=60, scale=0.1)
    o_direct, _ = fa.fwd(qd.detach(), kd.detach(), vd.detach(), causal=True, window_left=60, scale=0.1)
    (o * dod).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_direct)
    for t, r in zip((qd, kd, vd), ref):
        np.testing.assert_array_equal(t.grad.double().cpu().numpy(), r)
    grads, mag = oracle_grads(q, k, v, do, True, 60, 0.1)
    check_grads(ref, grads, mag, "bf16", 200, "autograd")
