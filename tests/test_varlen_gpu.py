"""GPU parity of the packed variable-length forward (``fa.fwd_varlen`` ->
``fa_fwd_varlen``) with the fp64 oracle ``attention_fwd_varlen``.

Tolerance: the forward's for 16-bit inputs (max |dO| <= 1e-2 and mean |dO|
<= 1e-3, scaled by max(1, |O_ref|) elementwise; max |dlse| <= 1e-3).  Rows
that see no key must give exactly o = 0 and lse = -inf.  With equal lengths
the packed path must reproduce the [B][H][N][d] forward bit for bit (same
tiles, same arithmetic).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from oracle import attention_fwd_varlen
from tests.gpu_util import announce, compare, to_dev
from workloads import VARLEN_WORKLOADS, make_varlen_inputs, round_to

pytestmark = pytest.mark.gpu


def _draw(seed, dtype, lq, lk, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = round_to(dtype, rng.standard_normal((int(cq[-1]), Hq, d), dtype=np.float32))
    k = round_to(dtype, rng.standard_normal((int(ck[-1]), Hkv, d), dtype=np.float32))
    v = round_to(dtype, rng.standard_normal((int(ck[-1]), Hkv, d), dtype=np.float32))
    return q, k, v, cq, ck


def run_varlen(q, k, v, cq, ck, causal, wl, scale, dtype, label, max_q=None, max_k=None):
    announce(f"varlen {label} q={q.shape} k={k.shape} B={len(cq) - 1} causal={causal} wl={wl}")
    mq = int(np.diff(cq).max(initial=0)) if max_q is None else max_q
    mk = int(np.diff(ck).max(initial=0)) if max_k is None else max_k
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o, lse = fa.fwd_varlen(qd, kd, vd, torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), mq, mk,
                           causal=causal, window_left=wl, scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(o, lse, q, k, v, cq, ck, causal, wl, scale, dtype, label):
    ro, rl = attention_fwd_varlen(q, k, v, cq, ck, causal, wl, scale)
    empty = np.isneginf(rl)                      # [Hq, total_q]
    e_rows = empty.T                             # [total_q, Hq]
    assert (o[e_rows] == 0).all() and np.isneginf(lse[empty]).all(), f"{label}: empty rows"
    assert np.isfinite(o).all() and np.isfinite(lse[~empty]).all(), f"{label}: non-finite output"
    if (~empty).any():
        compare(o[~e_rows], lse[~empty], ro[~e_rows], rl[~empty], dtype, label=label, scaled=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_self_attention_lengths(dtype, d):
    lens = [1, 0, 33, 64, 100, 129, 300, 257]
    for Hq, Hkv in [(4, 4), (8, 2)]:
        q, k, v, cq, ck = _draw(1600 + d + Hq, dtype, lens, lens, Hq, Hkv, d)
        for causal, wl in [(True, -1), (False, -1), (True, 40), (False, 17), (True, 0)]:
            label = f"self d={d} H={Hq}/{Hkv} causal={causal} wl={wl}"
            o, lse = run_varlen(q, k, v, cq, ck, causal, wl, d ** -0.5, dtype, label)
            check(o, lse, q, k, v, cq, ck, causal, wl, d ** -0.5, dtype, label)


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_fewer_and_more_queries_than_keys(d):
    lq = [5, 130, 1, 64, 200, 40]
    lk = [300, 131, 77, 64, 90, 0]     # Lq < Lk, Lq > Lk (empty rows), an empty key set
    q, k, v, cq, ck = _draw(1620 + d, "bf16", lq, lk, 8, 2, d)
    for causal, wl in [(True, -1), (False, -1), (True, 30), (False, 12)]:
        label = f"ragged d={d} causal={causal} wl={wl}"
        o, lse = run_varlen(q, k, v, cq, ck, causal, wl, d ** -0.5, "bf16", label)
        check(o, lse, q, k, v, cq, ck, causal, wl, d ** -0.5, "bf16", label)


def test_varlen_equal_lengths_match_the_batched_forward_bitwise():
    B, Hq, Hkv, N, d = 3, 8, 2, 700, 128
    q, k, v, cq, ck = _draw(1630, "bf16", [N] * B, [N] * B, Hq, Hkv, d)
    for causal, wl in [(True, -1), (False, 100)]:
        o, lse = run_varlen(q, k, v, cq, ck, causal, wl, 0.09, "bf16", "equal lengths")
        qb = q.reshape(B, N, Hq, d).transpose(0, 2, 1, 3)
        kb = k.reshape(B, N, Hkv, d).transpose(0, 2, 1, 3)
        vb = v.reshape(B, N, Hkv, d).transpose(0, 2, 1, 3)
        announce("varlen vs batched forward")
        ob, lb = fa.fwd(*(to_dev(np.ascontiguousarray(x), "bf16") for x in (qb, kb, vb)), causal=causal,
                        window_left=wl, scale=0.09)
        torch.cuda.synchronize()
        ob = ob.double().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * N, Hq, d)
        lb = lb.double().cpu().numpy().transpose(1, 0, 2).reshape(Hq, B * N)
        np.testing.assert_array_equal(o, ob)
        np.testing.assert_array_equal(lse, lb)


def test_varlen_offsets_past_the_tensors_are_clamped():
    """Offsets beyond the packed lengths are clamped: the call reads nothing
    outside the tensors and equals the call with the clamped offsets."""
    q, k, v, cq, ck = _draw(1640, "bf16", [50, 70], [50, 70], 4, 4, 64)
    bad_q, bad_k = cq.copy(), ck.copy()
    bad_q[-1] += 1000
    bad_k[-1] += 1000
    o1, l1 = run_varlen(q, k, v, bad_q, bad_k, True, -1, 0.125, "bf16", "offsets past the end", 1070, 1070)
    o2, l2 = run_varlen(q, k, v, cq, ck, True, -1, 0.125, "bf16", "clamped offsets", 1070, 1070)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_varlen_workload_every_sequence():
    """The full packed workload in the benchmark's launch configuration,
    every element of every sequence against the packed oracle (its worker
    threads each hold BLAS to one thread)."""
    from threadpoolctl import threadpool_limits
    w = VARLEN_WORKLOADS["varlen_causal_16"]
    q, k, v, cu = make_varlen_inputs(w)
    o, lse = run_varlen(q, k, v, cu, cu, w.causal, w.window_left, w.scale, w.dtype, "varlen_causal_16 full")
    with threadpool_limits(limits=1):
        check(o, lse, q, k, v, cu, cu, w.causal, w.window_left, w.scale, w.dtype, "varlen_causal_16 every sequence")


def test_varlen_rows_no_sequence_computes():
    """Rows past cu_seqlens_q[B] (and, with a max_seqlen_q below a
    sequence's length, that sequence's rows from max_seqlen_q on): the C call
    leaves the caller's buffers there untouched (a NaN fill survives bit for
    bit); buffers the binding allocates hold o = 0 and lse = -inf there.  The
    sequences within the stated maxima are computed as usual."""
    lq = [60, 200]
    q, k, v, cq, ck = _draw(1650, "bf16", lq, lq, 4, 2, 64)
    total_q = q.shape[0]
    pad = 37
    qp = np.concatenate([q, np.ones((pad,) + q.shape[1:], np.float32)])
    qd, kd, vd = (to_dev(x, "bf16") for x in (qp, k, v))
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    announce("varlen rows no sequence computes")
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((4, total_q + pad), float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd_varlen(qd, kd, vd, cqd, ckd, 128, 200, causal=True, scale=0.125, out=o, lse=lse)
    o2, l2 = fa.fwd_varlen(qd, kd, vd, cqd, ckd, 128, 200, causal=True, scale=0.125)
    torch.cuda.synchronize()
    o, lse, o2, l2 = (x.double().cpu().numpy() for x in (o, lse, o2, l2))
    untouched = np.zeros(total_q + pad, dtype=bool)
    untouched[60 + 128:total_q] = True        # second sequence's rows from max_seqlen_q on
    untouched[total_q:] = True                # rows no sequence owns
    assert np.isnan(o[untouched]).all() and np.isnan(lse[:, untouched]).all()
    assert (o2[untouched] == 0).all() and np.isneginf(l2[:, untouched]).all()
    assert np.isfinite(o[~untouched]).all() and np.isfinite(lse[:, ~untouched]).all()
    np.testing.assert_array_equal(o[~untouched], o2[~untouched])
    np.testing.assert_array_equal(lse[:, ~untouched], l2[:, ~untouched])
    # the first sequence (60 rows, within both maxima) is exact attention
    sub = np.array([0, 60], dtype=np.int32)
    check(o[:60], lse[:, :60], q[:60], k[:60], v[:60], sub, sub, True, -1, 0.125, "bf16", "first sequence")
