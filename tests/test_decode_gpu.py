"""GPU parity of attention against a key/value cache (``fa.fwd_kvcache``,
``fa.fwd_kvcache_paged`` -> ``fa_fwd_kvcache(_paged)``) with the fp64 cache
oracle.

Tolerance: as the forward's for 16-bit inputs (max |dO| <= 1e-2 and mean
|dO| <= 1e-3, scaled by max(1, |O_ref|) elementwise since rows that see few
keys have outputs of the size of V; max |dlse| <= 1e-3).  Rows that see no
key must give exactly o = 0 and lse = -inf.  Paged caches carry NaN in every
slot and page that no sequence owns, and -1 in unused table entries, so any
read outside a sequence shows up as a non-finite output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from oracle import attention_fwd_kvcache
from tests.gpu_util import announce, compare, to_dev
from workloads import DECODE_WORKLOADS, build_pages, make_decode_inputs, round_to

pytestmark = pytest.mark.gpu


def _draw(seed, dtype, B, Hq, Hkv, Nq, Nk, d, lens):
    rng = np.random.default_rng(seed)
    q = round_to(dtype, rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
    k = round_to(dtype, rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
    v = round_to(dtype, rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
    return q, k, v, np.asarray(lens, dtype=np.int32)


def check(o, lse, q, k, v, lens, causal, wl, scale, dtype, label):
    ro, rl = attention_fwd_kvcache(q, k, v, lens, causal, wl, scale)
    empty = np.isneginf(rl)
    assert (o[empty] == 0).all() and np.isneginf(lse[empty]).all(), f"{label}: empty rows"
    assert np.isfinite(o).all() and np.isfinite(lse[~empty]).all(), f"{label}: non-finite output"
    if (~empty).any():
        compare(o[~empty], lse[~empty], ro[~empty], rl[~empty], dtype, label=label, scaled=True)


def run_contig(q, k, v, lens, causal, wl, scale, dtype, splits, label):
    announce(f"kvcache {label} q={q.shape} k={k.shape} lens={list(lens)[:6]} causal={causal} wl={wl} splits={splits}")
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    sd = torch.from_numpy(lens).cuda()
    o, lse = fa.fwd_kvcache(qd, kd, vd, sd, causal=causal, window_left=wl, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def run_paged(q, k, v, lens, page_size, seed, causal, wl, scale, dtype, splits, label):
    announce(f"kvcache paged {label} q={q.shape} k={k.shape} page={page_size} causal={causal} wl={wl} splits={splits}")
    kp, vp, table = build_pages(k, v, lens, page_size, seed, fill=np.nan, spare_pages=3)
    qd, kd, vd = to_dev(q, dtype), to_dev(kp, dtype), to_dev(vp, dtype)
    td, sd = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    o, lse = fa.fwd_kvcache_paged(qd, kd, vd, td, sd, causal=causal, window_left=wl, scale=scale,
                                  num_splits=splits)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


# --- contiguous cache: lengths around tile edges, empty and short caches,
# row counts across the 32-row blocks, every mask, fixed and automatic splits

SHAPES = [
    # (Hq, Hkv, Nq, Nk, lens)
    (4, 2, 1, 100, [100, 1, 37, 64]),
    (8, 2, 3, 257, [257, 2, 0, 96]),
    (8, 1, 5, 64, [64, 32, 3, 5]),        # G * Nq = 40: two row blocks, the second partly filled
    (32, 8, 16, 600, [600, 17, 300, 33]),  # G * Nq = 64
    (2, 2, 40, 130, [130, 40, 41, 128]),   # Nq > 32 on its own
    (8, 1, 12, 200, [200, 150, 13, 0]),    # G * Nq = 96: three blocks
    (16, 1, 9, 160, [160, 31, 9, 100]),    # G * Nq = 144: five blocks, the last partly filled
    # an even block count of at least four: two blocks per wavefront
    (16, 2, 13, 200, [200, 77, 13, 1]),    # G * Nq = 104: four blocks, the last partly filled
    (8, 1, 22, 96, [96, 40, 22, 64]),      # G * Nq = 176: six blocks, the last half filled
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_kvcache_shapes(dtype, d, shape):
    Hq, Hkv, Nq, Nk, lens = SHAPES[shape]
    q, k, v, lens = _draw(1500 + shape + d, dtype, len(lens), Hq, Hkv, Nq, Nk, d, lens)
    scale = d ** -0.5
    for causal, wl in [(True, -1), (False, -1), (True, 20), (False, 7), (True, 0)]:
        for splits in (1, 3, 0):
            label = f"shape {shape} d={d} causal={causal} wl={wl} splits={splits}"
            o, lse = run_contig(q, k, v, lens, causal, wl, scale, dtype, splits, label)
            check(o, lse, q, k, v, lens, causal, wl, scale, dtype, label)


def test_kvcache_many_splits_and_determinism():
    """Splits beyond the tiles there are (empty splits), and the same split
    count twice gives the same bits."""
    q, k, v, lens = _draw(1520, "bf16", 2, 8, 2, 2, 700, 128, [700, 90])
    for splits in (2, 7, 40, 128):
        o, lse = run_contig(q, k, v, lens, True, -1, 0.09, "bf16", splits, f"splits={splits}")
        check(o, lse, q, k, v, lens, True, -1, 0.09, "bf16", f"splits={splits}")
    a = run_contig(q, k, v, lens, True, 100, 0.09, "bf16", 5, "determinism 1")
    b = run_contig(q, k, v, lens, True, 100, 0.09, "bf16", 5, "determinism 2")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_kvcache_null_lengths_and_no_lse():
    q, k, v, _ = _draw(1530, "f16", 2, 4, 4, 3, 200, 64, [0, 0])
    qd, kd, vd = (to_dev(x, "f16") for x in (q, k, v))
    announce("kvcache null lengths")
    o, lse = fa.fwd_kvcache(qd, kd, vd, None, causal=True, scale=0.125, num_splits=2, want_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    ro, _ = attention_fwd_kvcache(q, k, v, None, True, -1, 0.125)
    full = np.full(2, 200, dtype=np.int32)
    o2, l2 = run_contig(q, k, v, full, True, -1, 0.125, "f16", 2, "explicit full lengths")
    np.testing.assert_array_equal(o.double().cpu().numpy(), o2)
    check(o2, l2, q, k, v, full, True, -1, 0.125, "f16", "null lengths")
    assert np.abs(o2 - ro).max() < 1e-2


# --- paged cache ------------------------------------------------------------

@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_kvcache_paged(page_size, d):
    Nk = 4 * 256
    lens = [Nk, 1, 300, 0, 255, 257]
    q, k, v, lens = _draw(1540 + page_size + d, "bf16", len(lens), 8, 2, 2, Nk, d, lens)
    for causal, wl in [(True, -1), (False, 50)]:
        for splits in (1, 4, 0):
            label = f"page {page_size} d={d} causal={causal} wl={wl} splits={splits}"
            o, lse = run_paged(q, k, v, lens, page_size, 1540, causal, wl, d ** -0.5, "bf16", splits, label)
            check(o, lse, q, k, v, lens, causal, wl, d ** -0.5, "bf16", label)
            oc, lc = run_contig(q, k, v, lens, causal, wl, d ** -0.5, "bf16", splits, label + " contiguous")
            np.testing.assert_array_equal(o, oc)  # same tiles, same arithmetic
            np.testing.assert_array_equal(lse, lc)


@pytest.mark.parametrize("page_size", [16, 32])
def test_kvcache_paged_bad_page_index_reads_zeros(page_size):
    """A table entry outside [0, num_pages) inside a sequence reads as zeros:
    no fault, finite output (its keys score 0 and carry zero values)."""
    q, k, v, lens = _draw(1560, "bf16", 1, 4, 4, 1, 128, 64, [128])
    kp, vp, table = build_pages(k, v, lens, page_size, 1560)
    table[0, 1] = 10 ** 6
    kz, vz = k.copy(), v.copy()
    kz[:, :, page_size:2 * page_size] = 0
    vz[:, :, page_size:2 * page_size] = 0
    qd, kd, vd = to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16")
    announce("kvcache paged bad page index")
    o, lse = fa.fwd_kvcache_paged(qd, kd, vd, torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(),
                                  causal=True, scale=0.125, num_splits=1)
    torch.cuda.synchronize()
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), q, kz, vz, lens, True, -1, 0.125, "bf16",
          "bad page index")


# --- the decoding workloads at full size: every row -------------------------

@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_workload_full_size(name):
    w = DECODE_WORKLOADS[name]
    q, k, v, lens = make_decode_inputs(w)
    # the split count the benchmark launches with: chosen from the lengths
    splits = fa.kvcache_num_splits(lens, w.Hq, w.Hkv, w.Nq, w.Nk, w.causal, w.window_left)
    if w.page_size:
        o, lse = run_paged(q, k, v, lens, w.page_size, w.seed, w.causal, w.window_left, w.scale, w.dtype,
                           splits, f"{name} full")
    else:
        o, lse = run_contig(q, k, v, lens, w.causal, w.window_left, w.scale, w.dtype, splits, f"{name} full")
    check(o, lse, q, k, v, lens, w.causal, w.window_left, w.scale, w.dtype, f"{name} full, every row")
