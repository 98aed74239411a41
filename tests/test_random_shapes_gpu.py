"""Seeded random shapes through every entry point, each against the fp64
oracle at the bound its own parity module states.

The edge-case modules pick sizes around the tile edges by hand; here every
size is drawn: batch, head counts and GQA group, sequence length, head
dimension, mask (causal or not, a window of any width, none), the sign and
size of the softmax scale, packed sequence lengths (empty ones included),
cache lengths, page sizes and split counts.  Case i of each entry point
draws from its own seed (7000 + i forward, 7100 + i backward, 7200 + i FP8,
7300 + i and 7400 + i packed, 7500 + i cache), so a failure names a
reproducible case.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import attention_fwd
from tests import test_bwd_gpu as BW
from tests import test_bwd_varlen_gpu as BV
from tests import test_decode_gpu as DE
from tests import test_fp8_gpu as F8
from tests import test_varlen_gpu as VL
from tests.gpu_util import compare, run_gpu
from workloads import random_grad, random_inputs

pytestmark = pytest.mark.gpu


def _mask(rng, n):
    causal = bool(rng.integers(2))
    wl = -1 if rng.random() < 0.4 else int(rng.integers(0, n + 64))
    return causal, wl


def _scale(rng, d):
    s = d ** -0.5 * rng.uniform(0.25, 2.0)
    return float(np.float32(-s if rng.random() < 0.15 else s))


def _heads(rng):
    hkv = int(rng.integers(1, 4))
    return hkv * int(rng.choice([1, 2, 3, 4, 8])), hkv


@pytest.mark.parametrize("i", range(30))
def test_random_forward(i):
    rng = np.random.default_rng(7000 + i)
    dtype = ("bf16", "f16", "f32")[i % 3]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    Hq, Hkv = _heads(rng)
    N = int(rng.integers(1, 1001 if dtype == "f32" else 1501))
    causal, wl = _mask(rng, N)
    scale = _scale(rng, d)
    q, k, v = random_inputs(7000 + i, dtype, B, Hq, Hkv, N, d)
    label = f"random fwd {i}: B={B} H={Hq}/{Hkv} N={N} d={d} causal={causal} wl={wl} scale={scale:.4g}"
    o, lse = run_gpu(q, k, v, dtype, causal, wl, scale, label=label)
    ro, rl = attention_fwd(q, k, v, causal, wl, scale)
    compare(o, lse, ro, rl, dtype, label=label, scaled=True)


@pytest.mark.parametrize("i", range(12))
def test_random_backward(i):
    rng = np.random.default_rng(7100 + i)
    dtype = ("bf16", "f16")[i % 2]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    Hq, Hkv = _heads(rng)
    N = int(rng.integers(1, 501))
    causal, wl = _mask(rng, N)
    scale = _scale(rng, d)
    q, k, v = random_inputs(7100 + i, dtype, B, Hq, Hkv, N, d)
    do = random_grad(7150 + i, dtype, B, Hq, N, d)
    label = f"random bwd {i}: B={B} H={Hq}/{Hkv} N={N} d={d} causal={causal} wl={wl} scale={scale:.4g}"
    got = BW.run_bwd_gpu(q, k, v, do, dtype, causal, wl, scale, label)
    ref, mag = BW.oracle_grads(q, k, v, do, causal, wl, scale)
    BW.check_grads(got, ref, mag, dtype, N, label)


@pytest.mark.parametrize("i", range(10))
def test_random_fp8(i):
    rng = np.random.default_rng(7200 + i)
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    Hq, Hkv = _heads(rng)
    N = int(rng.integers(1, 1001))
    causal, wl = _mask(rng, N)
    scale = _scale(rng, d)
    b3, s3, deq = F8.quantize3(*random_inputs(7200 + i, "f32", B, Hq, Hkv, N, d))
    label = f"random fp8 {i}: B={B} H={Hq}/{Hkv} N={N} d={d} causal={causal} wl={wl} scale={scale:.4g}"
    o, lse = F8.run_fp8_gpu(b3, s3, causal, wl, scale, label)
    F8.check_fp8(o, lse, deq, causal, wl, scale, label)


def _lengths(rng, n_seq, hi):
    lens = rng.integers(0, hi + 1, size=n_seq)
    lens[rng.random(n_seq) < 0.15] = 0
    return [int(x) for x in lens]


@pytest.mark.parametrize("i", range(8))
def test_random_packed_forward(i):
    rng = np.random.default_rng(7300 + i)
    dtype = ("bf16", "f16")[i % 2]
    d = int(rng.choice([64, 128]))
    Hq, Hkv = _heads(rng)
    n_seq = int(rng.integers(1, 7))
    lk = _lengths(rng, n_seq, 700)
    lq = lk if rng.random() < 0.5 else _lengths(rng, n_seq, 700)
    causal, wl = _mask(rng, max(lk + lq))
    scale = _scale(rng, d)
    q, k, v, cq, ck = VL._draw(7300 + i, dtype, lq, lk, Hq, Hkv, d)
    label = f"random packed {i}: lq={lq} lk={lk} H={Hq}/{Hkv} d={d} causal={causal} wl={wl} scale={scale:.4g}"
    o, lse = VL.run_varlen(q, k, v, cq, ck, causal, wl, scale, dtype, label)
    VL.check(o, lse, q, k, v, cq, ck, causal, wl, scale, dtype, label)


@pytest.mark.parametrize("i", range(6))
def test_random_packed_backward(i):
    rng = np.random.default_rng(7400 + i)
    dtype = ("bf16", "f16")[i % 2]
    d = int(rng.choice([64, 128]))
    Hq, Hkv = _heads(rng)
    n_seq = int(rng.integers(1, 6))
    lk = _lengths(rng, n_seq, 400)
    lq = lk if rng.random() < 0.5 else _lengths(rng, n_seq, 400)
    causal, wl = _mask(rng, max(lk + lq))
    scale = _scale(rng, d)
    q, k, v, do, cq, ck = BV._draw(7400 + i, dtype, lq, lk, Hq, Hkv, d)
    label = f"random packed bwd {i}: lq={lq} lk={lk} H={Hq}/{Hkv} d={d} causal={causal} wl={wl}"
    got = BV.run(q, k, v, do, cq, ck, causal, wl, scale, dtype, label)
    BV.check(got, q, k, v, do, cq, ck, causal, wl, scale, dtype, label)


@pytest.mark.parametrize("i", range(12))
def test_random_kvcache(i):
    rng = np.random.default_rng(7500 + i)
    dtype = ("bf16", "f16")[i % 2]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 5))
    Hq, Hkv = _heads(rng)
    Nq = int(rng.integers(1, 17))
    Nk = int(rng.integers(1, 901))
    page = int(rng.choice([16, 32, 64, 96, 256]))
    paged = i % 2 == 1
    if paged:   # a paged cache's capacity is whole pages
        Nk = -(-Nk // page) * page
    lens = [int(x) for x in rng.integers(0, Nk + 1, size=B)]
    causal, wl = _mask(rng, Nk)
    scale = _scale(rng, d)
    splits = int(rng.choice([0, 1, int(rng.integers(2, 17))]))
    q, k, v, lens = DE._draw(7500 + i, dtype, B, Hq, Hkv, Nq, Nk, d, lens)
    label = (f"random cache {i}: B={B} H={Hq}/{Hkv} Nq={Nq} Nk={Nk} lens={list(lens)} d={d} causal={causal} "
             f"wl={wl} splits={splits}")
    if not paged:
        o, lse = DE.run_contig(q, k, v, lens, causal, wl, scale, dtype, splits, label)
    else:
        o, lse = DE.run_paged(q, k, v, lens, page, 7550 + i, causal, wl, scale, dtype, splits,
                              label + f" page={page}")
    DE.check(o, lse, q, k, v, lens, causal, wl, scale, dtype, label)
