"""GPU parity of the packed-sequence backward (``fa.bwd_varlen`` ->
``fa_bwd_varlen``) against the fp64 packed gradient oracle.

o and lse come from this library's packed forward, as a caller would pass
them; the bound per element is the fixed-length backward's (see
``test_bwd_gpu``), with the longest sequence as the number of summed terms.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_tiled_attention_04_amd as fa
from oracle import attention_bwd_varlen
from tests.gpu_util import announce, to_dev
from tests.test_bwd_gpu import check_grads, score_size
from workloads import round_to

pytestmark = pytest.mark.gpu


def _draw(seed, dtype, lq, lk, Hq, Hkv, d, extra_q=0, extra_k=0):
    rng = np.random.default_rng(seed)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    tq, tk = int(cq[-1]) + extra_q, int(ck[-1]) + extra_k
    q = round_to(dtype, rng.standard_normal((tq, Hq, d), dtype=np.float32))
    k = round_to(dtype, rng.standard_normal((tk, Hkv, d), dtype=np.float32))
    v = round_to(dtype, rng.standard_normal((tk, Hkv, d), dtype=np.float32))
    do = round_to(dtype, rng.standard_normal((tq, Hq, d), dtype=np.float32))
    return q, k, v, do, cq, ck


def run(q, k, v, do, cq, ck, causal, wl, scale, dtype, label, max_q=None, max_k=None, fill=None):
    announce(f"bwd varlen {label} q={q.shape} k={k.shape} B={len(cq) - 1} causal={causal} wl={wl}")
    mq = int(np.diff(cq).max(initial=0)) if max_q is None else max_q
    mk = int(np.diff(ck).max(initial=0)) if max_k is None else max_k
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, mq, mk, causal=causal, window_left=wl, scale=scale)
    grads = None
    if fill is not None:
        grads = {n: torch.full_like(t, fill) for n, t in (("dq", qd), ("dk", kd), ("dv", vd))}
    dq, dk, dv = fa.bwd_varlen(qd, kd, vd, o, lse, dod, cqd, ckd, mq, mk, causal=causal, window_left=wl,
                               scale=scale, **(grads or {}))
    torch.cuda.synchronize()
    return tuple(x.double().cpu().numpy() for x in (dq, dk, dv))


def check(got, q, k, v, do, cq, ck, causal, wl, scale, dtype, label):
    dq, dk, dv, mag = attention_bwd_varlen(q, k, v, do, cq, ck, causal, wl, scale, bounds=True)
    mag["score_size"] = score_size(q, k, scale)
    n = max(int(np.diff(cq).max(initial=1)), int(np.diff(ck).max(initial=1)))
    check_grads(got, (dq, dk, dv), mag, dtype, n, label)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_varlen_self_attention_lengths(dtype, d):
    lens = [1, 0, 33, 64, 100, 129, 300, 257]
    q, k, v, do, cq, ck = _draw(1700 + d, dtype, lens, lens, 8, 2, d)
    for causal, wl in [(True, -1), (False, -1), (True, 40), (False, 17), (True, 0)]:
        label = f"self d={d} causal={causal} wl={wl}"
        got = run(q, k, v, do, cq, ck, causal, wl, d ** -0.5, dtype, label)
        check(got, q, k, v, do, cq, ck, causal, wl, d ** -0.5, dtype, label)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_varlen_fewer_and_more_queries_than_keys(d):
    lq = [5, 130, 1, 64, 200, 40]
    lk = [300, 131, 77, 64, 90, 0]     # Lq < Lk, Lq > Lk (rows that see no key), an empty key set
    q, k, v, do, cq, ck = _draw(1720 + d, "bf16", lq, lk, 8, 2, d)
    for causal, wl in [(True, -1), (False, -1), (True, 30), (False, 12)]:
        label = f"ragged d={d} causal={causal} wl={wl}"
        got = run(q, k, v, do, cq, ck, causal, wl, d ** -0.5, "bf16", label)
        check(got, q, k, v, do, cq, ck, causal, wl, d ** -0.5, "bf16", label)


def test_bwd_varlen_equal_lengths_match_the_batched_backward_bitwise():
    B, Hq, Hkv, N, d = 3, 8, 2, 700, 128
    q, k, v, do, cq, ck = _draw(1730, "bf16", [N] * B, [N] * B, Hq, Hkv, d)
    for causal, wl in [(True, -1), (False, 100)]:
        got = run(q, k, v, do, cq, ck, causal, wl, 0.09, "bf16", "equal lengths")
        announce("bwd varlen vs batched backward")
        to_b = lambda x, H: np.ascontiguousarray(x.reshape(B, N, H, d).transpose(0, 2, 1, 3))  # noqa: E731
        qb, dob = to_dev(to_b(q, Hq), "bf16"), to_dev(to_b(do, Hq), "bf16")
        kb, vb = to_dev(to_b(k, Hkv), "bf16"), to_dev(to_b(v, Hkv), "bf16")
        ob, lb = fa.fwd(qb, kb, vb, causal=causal, window_left=wl, scale=0.09)
        ref = fa.bwd(qb, kb, vb, ob, lb, dob, causal=causal, window_left=wl, scale=0.09)
        torch.cuda.synchronize()
        for g, r, H in zip(got, ref, (Hq, Hkv, Hkv)):
            r = r.double().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * N, H, d)
            np.testing.assert_array_equal(g, r)


def test_bwd_varlen_offsets_past_the_tensors_are_clamped():
    """Offsets beyond the packed lengths are clamped: nothing outside the
    tensors is read or written, and the call equals the clamped one."""
    q, k, v, do, cq, ck = _draw(1740, "bf16", [50, 70], [50, 70], 4, 4, 64)
    bad_q, bad_k = cq.copy(), ck.copy()
    bad_q[-1] += 1000
    bad_k[-1] += 1000
    g1 = run(q, k, v, do, bad_q, bad_k, True, -1, 0.125, "bf16", "offsets past the end", 1070, 1070)
    g2 = run(q, k, v, do, cq, ck, True, -1, 0.125, "bf16", "clamped offsets", 1070, 1070)
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(a, b)


def test_bwd_varlen_rows_outside_every_sequence_are_untouched():
    lens = [70, 0, 129]
    q, k, v, do, cq, ck = _draw(1750, "f16", lens, lens, 4, 2, 128, extra_q=9, extra_k=5)
    got = run(q, k, v, do, cq, ck, True, -1, 0.1, "f16", "extra rows", fill=3.0)
    assert (got[0][cq[-1]:] == 3.0).all() and (got[1][ck[-1]:] == 3.0).all() and (got[2][ck[-1]:] == 3.0).all()
    check(tuple(g[:int(c[-1])] for g, c in zip(got, (cq, ck, ck))), q[:cq[-1]], k[:ck[-1]], v[:ck[-1]],
          do[:cq[-1]], cq, ck, True, -1, 0.1, "f16", "extra rows")


def test_differentiable_packed_attention_matches_fwd_and_bwd():
    """fa.attend_varlen under torch autograd gives the same bits as calling
    fwd_varlen and bwd_varlen directly."""
    lq, lk = [40, 0, 130, 7], [60, 5, 130, 3]
    q, k, v, do, cq, ck = _draw(1760, "bf16", lq, lk, 4, 2, 64)
    ref = run(q, k, v, do, cq, ck, True, 25, 0.12, "bf16", "autograd reference")
    qd, kd, vd = (to_dev(x, "bf16").requires_grad_() for x in (q, k, v))
    dod = to_dev(do, "bf16")
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    announce("autograd packed attention")
    o = fa.attend_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), causal=True, window_left=25, scale=0.12)
    o_direct, _ = fa.fwd_varlen(qd.detach(), kd.detach(), vd.detach(), cqd, ckd, max(lq), max(lk), causal=True,
                                window_left=25, scale=0.12)
    (o * dod).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_direct)
    for t, r in zip((qd, kd, vd), ref):
        np.testing.assert_array_equal(t.grad.double().cpu().numpy(), r)
