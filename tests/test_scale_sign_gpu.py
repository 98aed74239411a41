"""GPU parity for a zero or negative softmax scale, on every path that takes
one (forward in all three input types, backward, FP8 forward, decoding,
packed sequences), against the same fp64 oracles and bounds as the positive
scales.  scale * q.k with scale < 0 favours the keys least aligned with the
query; scale = 0 averages the visible V rows (lse = ln of their count).

The kernels take a row's maximum over the raw products and multiply by the
scale afterwards, so they apply a negative scale as |scale| on negated
queries: negation is exact, hence the forward at -c must equal the forward
at +c on -q bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from oracle import attention_fwd
from tests.gpu_util import announce, check_rounding_bound, compare, run_gpu, to_dev
from workloads import random_grad, random_inputs

pytestmark = pytest.mark.gpu

SCALES = [0.0, -0.0, -0.09, -0.125]
MASKS = [(False, -1), (True, -1), (True, 50), (False, 0)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", SCALES)
def test_forward_zero_and_negative_scale(dtype, d, scale):
    """The edge tests' input recipe and tolerance, plus the per-element
    rounding bound of the kernels' arithmetic."""
    q, k, v = random_inputs(2100 + d, dtype, 1, 4, 2, 300, d)
    for causal, wl in MASKS:
        label = f"fwd scale={scale} dtype={dtype} d={d} causal={causal} wl={wl}"
        o, lse = run_gpu(q, k, v, dtype, causal, wl, scale, label=label)
        ro, rl = attention_fwd(q, k, v, causal, wl, scale)
        compare(o, lse, ro, rl, dtype, label=label, scaled=True)
        check_rounding_bound(o, lse, q, k, v, causal, wl, scale, dtype, label=label)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forward_rounding_bound_larger_scores(dtype):
    """Inputs 1.5 times larger (peakier rows) at positive and negative
    scales: the per-element rounding bound holds on either sign."""
    q, k, v = random_inputs(2105, dtype, 1, 4, 2, 300, 128, mult=1.5)
    for scale in (0.125, -0.125):
        for causal, wl in MASKS:
            label = f"larger scores scale={scale} dtype={dtype} causal={causal} wl={wl}"
            o, lse = run_gpu(q, k, v, dtype, causal, wl, scale, label=label)
            check_rounding_bound(o, lse, q, k, v, causal, wl, scale, dtype, label=label)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_negative_scale_is_positive_scale_on_negated_queries(dtype):
    q, k, v = random_inputs(2110, dtype, 2, 4, 1, 257, 128)
    for causal, wl in [(True, -1), (False, 40)]:
        a = run_gpu(q, k, v, dtype, causal, wl, -0.1, label=f"-c dtype={dtype}")
        b = run_gpu(-q, k, v, dtype, causal, wl, 0.1, label=f"+c on -q dtype={dtype}")
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_backward_zero_and_negative_scale(dtype, scale):
    from tests.test_bwd_gpu import check_grads, oracle_grads, run_bwd_gpu
    q, k, v = random_inputs(2120, dtype, 1, 4, 2, 300, 128, mult=1.5)
    do = random_grad(2121, dtype, 1, 4, 300, 128)
    for causal, wl in MASKS:
        label = f"bwd scale={scale} dtype={dtype} causal={causal} wl={wl}"
        got = run_bwd_gpu(q, k, v, do, dtype, causal, wl, scale, label)
        ref, mag = oracle_grads(q, k, v, do, causal, wl, scale)
        check_grads(got, ref, mag, dtype, 300, label)


@pytest.mark.parametrize("scale", [0.0, -0.1])
def test_fp8_zero_and_negative_scale(scale):
    from tests.test_fp8_gpu import check_fp8, quantize3, run_fp8_gpu
    b3, s3, deq = quantize3(*random_inputs(2130, "f32", 1, 4, 2, 300, 128))
    for causal, wl in MASKS:
        label = f"fp8 scale={scale} causal={causal} wl={wl}"
        o, lse = run_fp8_gpu(b3, s3, causal, wl, scale, label)
        check_fp8(o, lse, deq, causal, wl, scale, label)


@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_decode_zero_and_negative_scale(scale):
    from tests.test_decode_gpu import _draw, check, run_contig, run_paged
    q, k, v, lens = _draw(2140, "bf16", 3, 8, 2, 3, 320, 128, [300, 0, 77])
    for causal, wl in [(True, -1), (False, -1), (True, 20)]:
        for splits in (1, 3):
            label = f"decode scale={scale} causal={causal} wl={wl} splits={splits}"
            o, lse = run_contig(q, k, v, lens, causal, wl, scale, "bf16", splits, label)
            check(o, lse, q, k, v, lens, causal, wl, scale, "bf16", label)
            op, lp = run_paged(q, k, v, lens, 32, 2140, causal, wl, scale, "bf16", splits, label + " paged")
            np.testing.assert_array_equal(op, o)
            np.testing.assert_array_equal(lp, lse)


@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_varlen_zero_and_negative_scale(scale):
    from tests.test_varlen_gpu import _draw, check, run_varlen
    lq, lk = [40, 0, 130, 7], [100, 5, 130, 3]
    q, k, v, cq, ck = _draw(2150, "f16", lq, lk, 4, 2, 64)
    for causal, wl in [(True, -1), (False, -1), (True, 30)]:
        label = f"varlen scale={scale} causal={causal} wl={wl}"
        o, lse = run_varlen(q, k, v, cq, ck, causal, wl, scale, "f16", label)
        check(o, lse, q, k, v, cq, ck, causal, wl, scale, "f16", label)


def test_zero_scale_averages_the_visible_values():
    """scale = 0, causal: row i's output is the mean of V rows 0..i exactly
    up to the output rounding, and lse is ln(i + 1)."""
    q, k, v = random_inputs(2160, "bf16", 1, 2, 2, 200, 64)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    announce("zero scale mean of visible rows")
    o, lse = fa.fwd(qd, kd, vd, causal=True, scale=0.0)
    torch.cuda.synchronize()
    want = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 201)[None, None, :, None]
    np.testing.assert_allclose(o.double().cpu().numpy(), want, rtol=2.0 ** -8, atol=1e-6)
    np.testing.assert_allclose(lse.double().cpu().numpy(), np.broadcast_to(np.log(np.arange(1, 201)), (1, 2, 200)),
                               rtol=0, atol=2e-6)
