"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (per input type): float32 1e-5 max abs on O and lse; float16 and
bfloat16 1e-2 max abs and 1e-3 mean abs on O, 1e-3 max abs on lse.  The
oracle is fed the same rounded inputs and answers in unrounded fp64.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention_fwd
from tests.gpu_util import announce, compare, run_gpu, to_dev

pytestmark = pytest.mark.gpu


def _oracle(q, k, v, causal, wl, scale, rows=None):
    return attention_fwd(q, k, v, causal, wl, scale, rows=rows)


# ---------------------------------------------------------------------------
# The five workloads.  Reduced shapes: every output compared; they span many
# tiles and end on a ragged tail.  Full shapes: every output too.

REDUCED = {
    "tiny_f32": dict(),
    "bf16_n1k_d64": dict(),
    "causal_8k": dict(B=1, Hq=2, Hkv=2, N=1000),
    "gqa_f16_4k": dict(B=1, Hq=8, Hkv=2, N=1500),
    "swa_32k": dict(B=1, Hq=2, Hkv=2, N=5000),
}


@pytest.mark.parametrize("name", W.ORDER)
def test_workload_all_outputs(name):
    w = W.WORKLOADS[name]
    q, k, v = W.make_inputs(w, **REDUCED[name])
    o, lse = run_gpu(q, k, v, w.dtype, w.causal, w.window_left, w.scale, label=f"{name} reduced")
    ro, rl = _oracle(q, k, v, w.causal, w.window_left, w.scale)
    compare(o, lse, ro, rl, w.dtype, label=f"{name} reduced {q.shape}")


@pytest.mark.parametrize("name", ["causal_8k", "gqa_f16_4k", "swa_32k"])
def test_workload_full_size_every_element(name):
    """The full-size workloads in the launch configuration the benchmark
    times, every output element against the oracle (its worker threads each
    hold BLAS to one thread)."""
    from threadpoolctl import threadpool_limits
    w = W.WORKLOADS[name]
    q, k, v = W.make_inputs(w)
    o, lse = run_gpu(q, k, v, w.dtype, w.causal, w.window_left, w.scale, label=f"{name} full")
    with threadpool_limits(limits=1):
        ro, rl = attention_fwd(q, k, v, w.causal, w.window_left, w.scale, threads=len(os.sched_getaffinity(0)))
    compare(o, lse, ro, rl, w.dtype, label=f"{name} full, every element")


# ---------------------------------------------------------------------------
# Edge shapes: sequence lengths around the tile sizes, both head dims, all
# three input types, GQA groupings, every mask combination.

MASKS = [(False, -1), (True, -1), (False, 0), (True, 0), (True, 1), (False, 63), (True, 64), (True, 200)]


def _edge_cases():
    cases = []
    i = 0
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for N in (1, 17, 64, 129, 1000):
                for causal, wl in MASKS:
                    if N == 1000 and (causal, wl) not in [(False, -1), (True, -1), (True, 200), (False, 0)]:
                        continue
                    heads = [(1, 1), (4, 2), (6, 1)][i % 3]
                    i += 1
                    cases.append((dtype, d, N, heads[0], heads[1], causal, wl))
    return cases


@pytest.mark.parametrize("dtype,d,N,Hq,Hkv,causal,wl", _edge_cases())
def test_edge_shapes(dtype, d, N, Hq, Hkv, causal, wl):
    q, k, v = W.random_inputs(1000 + N + d, dtype, 2 if N < 200 else 1, Hq, Hkv, N, d)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_gpu(q, k, v, dtype, causal, wl, scale, label="edge")
    ro, rl = _oracle(q, k, v, causal, wl, scale)
    compare(o, lse, ro, rl, dtype, label=f"edge N={N} d={d} H={Hq}/{Hkv} causal={causal} wl={wl}",
            scaled=True)


@pytest.mark.parametrize("wl", [0, 1, 63, 64, 127, 128, 129, 298, 299, 4096])
@pytest.mark.parametrize("causal", [False, True])
def test_window_sizes(wl, causal):
    q, k, v = W.random_inputs(77, "bf16", 1, 2, 2, 300, 128)
    o, lse = run_gpu(q, k, v, "bf16", causal, wl, 0.088, label="window")
    ro, rl = _oracle(q, k, v, causal, wl, 0.088)
    compare(o, lse, ro, rl, "bf16", label=f"window wl={wl} causal={causal}", scaled=True)


def test_large_scores_fp16_outlier():
    """Scores far from zero (one channel scaled up): the running max must
    rescale correctly; the oracle decides."""
    q, k, v = W.random_inputs(78, "f16", 1, 4, 1, 700, 128)
    k[..., 5] *= 16.0
    q[..., 5] *= 4.0
    o, lse = run_gpu(q, k, v, "f16", True, -1, 0.088, label="outlier")
    ro, rl = _oracle(q, k, v, True, -1, 0.088)
    compare(o, lse, ro, rl, "f16", label="large scores")


# ---------------------------------------------------------------------------
# Properties that hold at any size.

def _fwd_dev(qd, kd, vd, causal=False, wl=-1, scale=0.1, want_lse=True):
    import exact_tiled_attention_04_amd as fa
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window_left=wl, scale=scale, want_lse=want_lse)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("name", ["causal_8k", "swa_32k"])
def test_deterministic_bitwise(name):
    w = W.WORKLOADS[name]
    q, k, v = W.make_inputs(w, B=1, Hq=4, Hkv=4, N=4096)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    announce(f"determinism {name}")
    o1, l1 = _fwd_dev(qd, kd, vd, w.causal, w.window_left, w.scale)
    o2, l2 = _fwd_dev(qd, kd, vd, w.causal, w.window_left, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_equals_mha_with_repeated_kv_bitwise():
    q, k, v = W.random_inputs(81, "bf16", 2, 8, 2, 777, 128)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    qd = to_dev(q, "bf16")
    announce("gqa vs mha")
    for causal, wl in [(False, -1), (True, -1), (True, 100)]:
        o1, l1 = _fwd_dev(qd, to_dev(k, "bf16"), to_dev(v, "bf16"), causal, wl, 0.09)
        o2, l2 = _fwd_dev(qd, to_dev(kr, "bf16"), to_dev(vr, "bf16"), causal, wl, 0.09)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (causal, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_mask_perturbation_bitwise(dtype):
    """Rows i <= i0 must not change when keys/values j > i0 are overwritten."""
    N, i0 = 640, 300
    q, k, v = W.random_inputs(82, dtype, 1, 2, 2, N, 128)
    announce(f"causal perturbation {dtype}")
    o1, l1 = _fwd_dev(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), True, -1, 0.09)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i0 + 1:] = 3000.0
    v2[:, :, i0 + 1:] = -5000.0
    o2, l2 = _fwd_dev(to_dev(q, dtype), to_dev(k2, dtype), to_dev(v2, dtype), True, -1, 0.09)
    assert torch.equal(o1[:, :, :i0 + 1], o2[:, :, :i0 + 1])
    assert torch.equal(l1[:, :, :i0 + 1], l2[:, :, :i0 + 1])
    assert not torch.equal(o1[:, :, i0 + 1:], o2[:, :, i0 + 1:])


@pytest.mark.parametrize("causal", [False, True])
def test_window_mask_perturbation_bitwise(causal):
    """Rows i >= i0 with window wl never see keys j < i0 - wl."""
    N, wl, i0 = 700, 130, 450
    q, k, v = W.random_inputs(83, "bf16", 1, 2, 2, N, 64)
    announce("window perturbation")
    o1, l1 = _fwd_dev(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), causal, wl, 0.12)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :i0 - wl] = 2000.0
    v2[:, :, :i0 - wl] = 7000.0
    o2, l2 = _fwd_dev(to_dev(q, "bf16"), to_dev(k2, "bf16"), to_dev(v2, "bf16"), causal, wl, 0.12)
    assert torch.equal(o1[:, :, i0:], o2[:, :, i0:])
    assert torch.equal(l1[:, :, i0:], l2[:, :, i0:])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_window_zero_returns_v(dtype):
    """window_left = 0 with causal: each query sees only its own key, so O = V.
    For 16-bit outputs this is exact (the weight is 1 up to a few fp32 ulps,
    far below half an output ulp); for fp32 it holds to a few ulps."""
    q, k, v = W.random_inputs(84, dtype, 1, 3, 3, 333, 64)
    announce(f"wl=0 {dtype}")
    vd = to_dev(v, dtype)
    o, lse = _fwd_dev(to_dev(q, dtype), to_dev(k, dtype), vd, True, 0, 0.2)
    if dtype == "f32":
        torch.testing.assert_close(o, vd, rtol=1e-6, atol=1e-7)
    else:
        assert torch.equal(o, vd)
    ref = 0.2 * np.einsum("bhnd,bhnd->bhn", q.astype(np.float64), k.astype(np.float64))
    assert np.abs(lse.double().cpu().numpy() - ref).max() <= 1e-4


def test_output_guard_bands_intact():
    """Sentinels around o and lse survive, at a ragged N."""
    B, H, N, d = 1, 3, 777, 128
    q, k, v = W.random_inputs(85, "bf16", B, H, H, N, d)
    pad = 4096
    o_buf = torch.full((2 * pad + B * H * N * d,), 12345.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((2 * pad + B * H * N,), -777.0, dtype=torch.float32, device="cuda")
    o = o_buf[pad:pad + B * H * N * d].view(B, H, N, d)
    lse = l_buf[pad:pad + B * H * N].view(B, H, N)
    import exact_tiled_attention_04_amd as fa
    announce("guard bands")
    fa.fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o_buf[:pad] == 12345.0).all()) and bool((o_buf[-pad:] == 12345.0).all())
    assert bool((l_buf[:pad] == -777.0).all()) and bool((l_buf[-pad:] == -777.0).all())
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())


def test_no_device_allocation_at_32k():
    """The library allocates nothing: device free memory is the same before and
    after a call at N = 32768 (where the score matrix would be 128 GiB fp32)."""
    w = W.WORKLOADS["swa_32k"]
    shape = (w.B, w.Hq, w.N, w.d)
    qd = torch.randn(shape, device="cuda", dtype=torch.bfloat16)
    kd = torch.randn(shape, device="cuda", dtype=torch.bfloat16)
    vd = torch.randn(shape, device="cuda", dtype=torch.bfloat16)
    o = torch.empty_like(qd)
    lse = torch.empty(shape[:3], device="cuda", dtype=torch.float32)
    import exact_tiled_attention_04_amd as fa
    announce("no allocation at 32k")
    fa.fwd(qd, kd, vd, causal=True, window_left=w.window_left, out=o, lse=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    fa.fwd(qd, kd, vd, causal=True, window_left=w.window_left, out=o, lse=lse)
    fa.fwd(qd, kd, vd, causal=False, window_left=-1, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_side_stream_and_no_lse():
    q, k, v = W.random_inputs(86, "bf16", 1, 4, 4, 500, 128)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    announce("side stream")
    o_ref, l_ref = _fwd_dev(qd, kd, vd, True, -1, 0.09)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    import exact_tiled_attention_04_amd as fa
    with torch.cuda.stream(s):
        o2, l2 = fa.fwd(qd, kd, vd, causal=True, scale=0.09)
        o3, l3 = fa.fwd(qd, kd, vd, causal=True, scale=0.09, want_lse=False)
    s.synchronize()
    assert l3 is None
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref) and torch.equal(o3, o_ref)


def test_errors_raise_and_write_nothing():
    import exact_tiled_attention_04_amd as fa
    q = torch.zeros((1, 3, 64, 64), device="cuda", dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 64, 64), device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 5.0)
    announce("error path")
    with pytest.raises(fa.FaError) as ei:
        fa.fwd(q, k, k, out=o)
    assert ei.value.status == -1
    q2 = torch.zeros((1, 2, 64, 96), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(fa.FaError) as ei:
        fa.fwd(q2, q2, q2)
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert bool((o == 5.0).all())


def test_empty_sequence_is_noop():
    import exact_tiled_attention_04_amd as fa
    q = torch.zeros((2, 2, 0, 128), device="cuda", dtype=torch.bfloat16)
    o, lse = fa.fwd(q, q, q, causal=True)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (2, 2, 0)
