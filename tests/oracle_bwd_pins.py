"""Pins for the attention-gradient oracle: each takes a function
bwd(q, k, v, do, causal, window_left, scale) -> (dq, dk, dv) in fp64 and
asserts a fact fixed by something other than the function itself:

- central finite differences of the *forward* oracle (the definition of a
  gradient, independent of any backward formula);
- torch's float64 autograd through a plainly written softmax attention (a
  library routine);
- closed forms: identical keys make the probabilities independent of the
  query (dQ = 0); one key makes dQ = dK = 0 and dV = dO; rows of P sum to one
  (sum_j dV_j = sum_i dO_i) and rows of dS sum to zero (sum_j dK_j = 0);
- linearity in the upstream gradient and equivariance under a permutation of
  the keys (no mask).

Pins for the packed-sequence gradients take bwd_varlen(q, k, v, do, cu_q,
cu_k, causal=, window_left=, scale=): central finite differences of the
packed forward oracle (sequences with fewer, as many and more queries than
keys, rows that see no key, a sequence with no queries), and, for equal
lengths, the fixed-length gradients above sequence by sequence.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention_bwd, attention_fwd, attention_fwd_varlen
from workloads import random_inputs

MASKS = [(False, -1), (True, -1), (False, 0), (False, 3), (True, 0), (True, 2), (True, 5)]


def _rand_do(seed, B, Hq, N, d):
    return np.random.default_rng(seed).standard_normal((B, Hq, N, d))


def pin_bwd_finite_differences(bwd):
    """dL/dx for L = sum(dO * O(q, k, v)), by central differences of the
    forward oracle, element by element."""
    shapes = [(1, 2, 1, 5, 3), (1, 2, 2, 4, 4), (2, 4, 2, 6, 2)]
    masks = [(False, -1), (True, -1), (True, 1), (False, 2)]
    h = 1e-5
    for si, (B, Hq, Hkv, N, d) in enumerate(shapes):
        q, k, v = (x.astype(np.float64) for x in random_inputs(300 + si, "f32", B, Hq, Hkv, N, d))
        do = _rand_do(400 + si, B, Hq, N, d)
        scale = 0.7
        for causal, wl in masks:
            def loss(qq, kk, vv):
                o, _ = attention_fwd(qq, kk, vv, causal, wl, scale, threads=1)
                return float((o * do).sum())
            dq, dk, dv = bwd(q, k, v, do, causal, wl, scale)
            for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
                num = np.zeros_like(x)
                for idx in np.ndindex(x.shape):
                    xp = x.copy()
                    xp[idx] += h
                    xm = x.copy()
                    xm[idx] -= h
                    args_p = {"q": q, "k": k, "v": v}
                    args_m = dict(args_p)
                    args_p[name], args_m[name] = xp, xm
                    num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                                loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
                np.testing.assert_allclose(g, num, rtol=0, atol=2e-8,
                                           err_msg=f"d{name} shape={B,Hq,Hkv,N,d} causal={causal} wl={wl}")


def _torch_grads(q, k, v, do, causal, wl, scale):
    import torch
    qt, kt, vt = (torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True) for x in (q, k, v))
    dot = torch.from_numpy(np.asarray(do, dtype=np.float64))
    N = qt.shape[2]
    allow = torch.ones(N, N, dtype=torch.bool)
    if causal:
        allow = allow.tril()
    if wl >= 0:
        allow = allow & torch.ones(N, N, dtype=torch.bool).triu(-wl)
    g = qt.shape[1] // kt.shape[1]
    kr = kt.repeat_interleave(g, dim=1)
    vr = vt.repeat_interleave(g, dim=1)
    s = torch.matmul(qt, kr.transpose(-1, -2)) * scale
    s = s.masked_fill(~allow, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vr)
    o.backward(dot)
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_bwd_torch_autograd(bwd):
    shapes = [(1, 1, 1, 1, 4), (2, 2, 2, 7, 8), (1, 4, 2, 13, 16), (1, 6, 2, 33, 8), (1, 2, 1, 64, 32)]
    for si, (B, Hq, Hkv, N, d) in enumerate(shapes):
        q, k, v = random_inputs(500 + si, "f32", B, Hq, Hkv, N, d)
        do = _rand_do(600 + si, B, Hq, N, d)
        scale = 0.37 if si % 2 else 1.0 / math.sqrt(d)
        for causal, wl in MASKS:
            got = bwd(q, k, v, do, causal, wl, scale)
            ref = _torch_grads(q, k, v, do, causal, wl, scale)
            for name, a, b in zip(("dq", "dk", "dv"), got, ref):
                np.testing.assert_allclose(a, b, rtol=0, atol=1e-11,
                                           err_msg=f"{name} shape={B,Hq,Hkv,N,d} causal={causal} wl={wl}")


def _visible(N, causal, wl):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), dtype=bool)
    if causal:
        vis &= j <= i
    if wl >= 0:
        vis &= j >= i - wl
    return vis


def pin_bwd_equal_keys(bwd):
    """Every key row equal: each query's probabilities are uniform over its
    visible keys whatever the query, so dQ = 0, and
    dV_j = sum over the group's heads and the rows i that see j of dO_i / n_i."""
    B, Hq, Hkv, N, d = 1, 4, 2, 9, 5
    q, k, v = random_inputs(700, "f32", B, Hq, Hkv, N, d)
    k = np.repeat(k[:, :, :1, :], N, axis=2)
    do = _rand_do(701, B, Hq, N, d)
    for causal, wl in MASKS:
        dq, dk, dv = bwd(q, k, v, do, causal, wl, 0.9)
        np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-12, err_msg=f"dq causal={causal} wl={wl}")
        vis = _visible(N, causal, wl).astype(np.float64)
        W = vis / vis.sum(axis=1, keepdims=True)          # uniform rows
        G = Hq // Hkv
        for hk in range(Hkv):
            want = sum(W.T @ do[0, hk * G + g] for g in range(G))
            np.testing.assert_allclose(dv[0, hk], want, rtol=0, atol=1e-12, err_msg=f"dv causal={causal} wl={wl}")


def pin_bwd_single_key(bwd):
    """N = 1: P = [[1]], so dV = dO (summed over the group), dQ = dK = 0."""
    q, k, v = random_inputs(710, "f32", 2, 6, 3, 1, 8)
    do = _rand_do(711, 2, 6, 1, 8)
    dq, dk, dv = bwd(q, k, v, do, True, 0, 0.5)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, do.reshape(2, 3, 2, 1, 8).sum(axis=2), rtol=0, atol=1e-12)


def pin_bwd_sum_rules(bwd):
    """Rows of P sum to 1: sum_j dV_j = sum over the group and rows of dO_i.
    Rows of dS sum to 0: sum_j dK_j = 0."""
    B, Hq, Hkv, N, d = 2, 6, 3, 17, 6
    q, k, v = random_inputs(720, "f32", B, Hq, Hkv, N, d)
    do = _rand_do(721, B, Hq, N, d)
    G = Hq // Hkv
    for causal, wl in MASKS:
        dq, dk, dv = bwd(q, k, v, do, causal, wl, 0.6)
        want = do.reshape(B, Hkv, G, N, d).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), want, rtol=0, atol=1e-11, err_msg=f"causal={causal} wl={wl}")
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-11, err_msg=f"causal={causal} wl={wl}")


def pin_bwd_linearity(bwd):
    B, Hq, Hkv, N, d = 1, 2, 1, 11, 4
    q, k, v = random_inputs(730, "f32", B, Hq, Hkv, N, d)
    d1 = _rand_do(731, B, Hq, N, d)
    d2 = _rand_do(732, B, Hq, N, d)
    for causal, wl in [(False, -1), (True, 3)]:
        g1 = bwd(q, k, v, d1, causal, wl, 0.8)
        g2 = bwd(q, k, v, d2, causal, wl, 0.8)
        g12 = bwd(q, k, v, d1 + 2 * d2, causal, wl, 0.8)
        for a, b, c in zip(g1, g2, g12):
            np.testing.assert_allclose(c, a + 2 * b, rtol=0, atol=1e-11)


def pin_bwd_key_permutation(bwd):
    """Without a mask, permuting the keys (with their values) permutes dK and
    dV the same way and leaves dQ unchanged."""
    B, Hq, Hkv, N, d = 1, 4, 2, 10, 3
    q, k, v = random_inputs(740, "f32", B, Hq, Hkv, N, d)
    do = _rand_do(741, B, Hq, N, d)
    perm = np.random.default_rng(742).permutation(N)
    dq, dk, dv = bwd(q, k, v, do, False, -1, 0.5)
    dq2, dk2, dv2 = bwd(q, k[:, :, perm], v[:, :, perm], do, False, -1, 0.5)
    np.testing.assert_allclose(dq2, dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk2, dk[:, :, perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv2, dv[:, :, perm], rtol=0, atol=1e-12)


def pin_bwd_zero_and_negative_scale(bwd):
    """scale = 0: P is uniform over the visible keys whatever Q and K are, so
    dQ = dK = 0 and dV_j = sum over the group and the rows i that see j of
    dO_i / n_i.  scale < 0: central finite differences of the forward oracle."""
    B, Hq, Hkv, N, d = 1, 4, 2, 7, 3
    q, k, v = (x.astype(np.float64) for x in random_inputs(750, "f32", B, Hq, Hkv, N, d))
    do = _rand_do(751, B, Hq, N, d)
    G = Hq // Hkv
    for causal, wl in MASKS:
        dq, dk, dv = bwd(q, k, v, do, causal, wl, 0.0)
        np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-13)
        vis = _visible(N, causal, wl).astype(np.float64)
        W = vis / vis.sum(axis=1, keepdims=True)
        for hk in range(Hkv):
            want = sum(W.T @ do[0, hk * G + g] for g in range(G))
            np.testing.assert_allclose(dv[0, hk], want, rtol=0, atol=1e-12)
    h = 1e-5
    for causal, wl in [(False, -1), (True, 2)]:
        scale = -0.8

        def loss(qq, kk, vv):
            o, _ = attention_fwd(qq, kk, vv, causal, wl, scale, threads=1)
            return float((o * do).sum())
        grads = bwd(q, k, v, do, causal, wl, scale)
        for name, x, g in zip("qkv", (q, k, v), grads):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                xp = x.copy()
                xp[idx] += h
                xm = x.copy()
                xm[idx] -= h
                args_p[name], args_m[name] = xp, xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                            loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=f"d{name} scale={scale} causal={causal}")


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_zero_and_negative_scale, pin_bwd_torch_autograd, pin_bwd_equal_keys, pin_bwd_single_key,
                pin_bwd_sum_rules, pin_bwd_linearity, pin_bwd_key_permutation]


# ---------------------------------------------------------------------------
# Packed sequences of different lengths

def pin_varlen_bwd_finite_differences(bwd_varlen):
    """dL/dx for L = sum(dO * O) of the packed forward oracle, by central
    differences, element by element; query rows stand at the end of their
    sequence's keys, and rows that see no key (more queries than keys under
    a causal mask) have o = 0, so no gradient."""
    lens = [(2, 4), (3, 3), (3, 1), (0, 2)]  # (queries, keys) per sequence
    cq = np.cumsum([0] + [a for a, _ in lens])
    ck = np.cumsum([0] + [b for _, b in lens])
    Hq, Hkv, d = 2, 1, 3
    rng = np.random.default_rng(470)
    q = rng.standard_normal((cq[-1], Hq, d))
    k = rng.standard_normal((ck[-1], Hkv, d))
    v = rng.standard_normal((ck[-1], Hkv, d))
    do = rng.standard_normal((cq[-1], Hq, d))
    scale, h = 0.8, 1e-5
    for causal, wl in [(False, -1), (True, -1), (True, 1), (False, 0)]:
        def loss(qq, kk, vv):
            o, _ = attention_fwd_varlen(qq, kk, vv, cq, ck, causal, wl, scale, threads=1)
            return float((o * do).sum())
        dq, dk, dv = bwd_varlen(q, k, v, do, cq, ck, causal=causal, window_left=wl, scale=scale)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                xp = x.copy()
                xp[idx] += h
                xm = x.copy()
                xm[idx] -= h
                args_p[name], args_m[name] = xp, xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                            loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=f"d{name} causal={causal} wl={wl}")


def pin_varlen_bwd_equal_lengths(bwd_varlen):
    """Equal query and key lengths: each sequence's gradients are the
    fixed-length gradients of that sequence alone (GQA, every mask kind)."""
    lens = [5, 1, 7, 3]
    cu = np.cumsum([0] + lens)
    Hq, Hkv, d = 4, 2, 4
    rng = np.random.default_rng(471)
    q = rng.standard_normal((cu[-1], Hq, d))
    k = rng.standard_normal((cu[-1], Hkv, d))
    v = rng.standard_normal((cu[-1], Hkv, d))
    do = rng.standard_normal((cu[-1], Hq, d))
    for causal, wl in MASKS:
        dq, dk, dv = bwd_varlen(q, k, v, do, cu, cu, causal=causal, window_left=wl, scale=0.6)
        for b in range(len(lens)):
            a, z = cu[b], cu[b + 1]
            per = lambda x: x[a:z].transpose(1, 0, 2)[None]  # noqa: E731  [1, H, L, d]
            rq, rk, rv = attention_bwd(per(q), per(k), per(v), per(do), causal, wl, 0.6, threads=1)
            for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
                np.testing.assert_allclose(got[a:z].transpose(1, 0, 2), ref[0], rtol=0, atol=1e-12,
                                           err_msg=f"{name} sequence {b} causal={causal} wl={wl}")


ALL_VARLEN_BWD_PINS = [pin_varlen_bwd_finite_differences, pin_varlen_bwd_equal_lengths]
