"""Pins for the exact-attention oracle: checks against things other than the
oracle itself (hand-worked values, closed forms, invariants, brute force, and
torch's CPU scaled-dot-product attention in float64).

Each pin takes an attention callable ``fwd(q, k, v, causal, window_left,
scale) -> (o, lse)`` on numpy arrays, and raises AssertionError when the
callable disagrees.  ``tests/test_oracle.py`` runs every pin on the oracle, and
also on copies of the oracle with planted mistakes, each of which must fail at
least one pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from workloads import random_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")

MASKS = [(False, -1), (True, -1), (False, 0), (False, 3), (True, 0), (True, 2), (True, 5)]


def _num(x):
    """Parse a hand-worked value: a number, 'p/q', 'lnA', or 'ClnA'."""
    if isinstance(x, (int, float)):
        return float(x)
    s = x.strip()
    if "ln" in s:
        coef, arg = s.split("ln")
        return (float(coef) if coef else 1.0) * math.log(float(arg))
    return float(Fraction(s))


def _arr(nested):
    return np.vectorize(_num, otypes=[np.float64])(np.array(nested, dtype=object))


def pin_hand_worked(fwd):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v = _arr(c["q"]), _arr(c["k"]), _arr(c["v"])
        o, lse = fwd(q, k, v, c["causal"], c["window_left"], c["scale"])
        np.testing.assert_allclose(o, _arr(c["o"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse, _arr(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])


def _torch_reference(q, k, v, causal, wl, scale):
    """torch's float64 CPU attention with a mask built from tril/triu."""
    import torch
    import torch.nn.functional as F
    qt, kt, vt = (torch.from_numpy(np.asarray(x, dtype=np.float64)) for x in (q, k, v))
    N = qt.shape[2]
    allow = torch.ones(N, N, dtype=torch.bool)
    if causal:
        allow = allow.tril()
    if wl >= 0:
        allow = allow & torch.ones(N, N, dtype=torch.bool).triu(-wl)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allow, scale=scale,
                                       enable_gqa=qt.shape[1] != kt.shape[1])
    g = qt.shape[1] // kt.shape[1]
    kr = kt.repeat_interleave(g, dim=1)
    s = torch.matmul(qt, kr.transpose(-1, -2)) * scale
    s = s.masked_fill(~allow, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def pin_torch_sdpa(fwd):
    shapes = [(1, 1, 1, 1, 4), (2, 2, 2, 7, 8), (1, 4, 2, 13, 16), (1, 6, 2, 33, 8), (1, 2, 1, 64, 32)]
    for si, (B, Hq, Hkv, N, d) in enumerate(shapes):
        q, k, v = random_inputs(100 + si, "f32", B, Hq, Hkv, N, d)
        scale = 0.37 if si % 2 else 1.0 / math.sqrt(d)
        for causal, wl in MASKS:
            o, lse = fwd(q, k, v, causal, wl, scale)
            ro, rl = _torch_reference(q, k, v, causal, wl, scale)
            np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12,
                                       err_msg=f"o shape={B,Hq,Hkv,N,d} causal={causal} wl={wl}")
            np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12,
                                       err_msg=f"lse shape={B,Hq,Hkv,N,d} causal={causal} wl={wl}")


def pin_rows_are_probabilities(fwd):
    """With V = identity (d = N), row i of O is row i of P: entries are
    non-negative, sum to 1, and are exactly zero on masked keys."""
    N = 9
    q, k, _ = random_inputs(7, "f32", 1, 2, 1, N, N)
    v = np.eye(N, dtype=np.float64)[None, None].repeat(1, axis=1)
    for causal, wl in MASKS:
        P, _ = fwd(q, k, v, causal, wl, 0.5)
        P = P[0]
        assert (P >= 0).all()
        np.testing.assert_allclose(P.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
        for i in range(N):
            for j in range(N):
                hidden = (causal and j > i) or (wl >= 0 and j < i - wl)
                if hidden:
                    assert P[:, i, j].max() == 0.0, (causal, wl, i, j)
                else:
                    assert P[:, i, j].min() > 0.0, (causal, wl, i, j)


def pin_shift_invariance(fwd):
    """Adding one vector u to every key row adds scale*<q_i, u> to every score
    of row i: P and O are unchanged and lse_i moves by exactly that amount."""
    B, Hq, Hkv, N, d = 1, 4, 2, 19, 8
    q, k, v = random_inputs(11, "f32", B, Hq, Hkv, N, d)
    u = np.linspace(-1.5, 2.0, d)
    scale = 0.3
    for causal, wl in MASKS:
        o0, l0 = fwd(q, k, v, causal, wl, scale)
        o1, l1 = fwd(q, k.astype(np.float64) + u, v, causal, wl, scale)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-11)
        np.testing.assert_allclose(l1 - l0, scale * (q.astype(np.float64) @ u), rtol=0, atol=1e-11)


def _visible(N, causal, wl):
    return [[j for j in range(N) if not ((causal and j > i) or (wl >= 0 and j < i - wl))]
            for i in range(N)]


def pin_all_equal_keys(fwd):
    """Every key equal: all visible scores tie, so O_i is the mean of the
    visible V rows and lse_i = scale*<q_i, k> + ln(n_i)."""
    B, Hq, Hkv, N, d = 1, 2, 1, 17, 4
    q, _, v = random_inputs(12, "f32", B, Hq, Hkv, N, d)
    kvec = np.array([0.5, -1.0, 2.0, 0.25])
    k = np.broadcast_to(kvec, (B, Hkv, N, d)).copy()
    scale = 0.7
    for causal, wl in MASKS:
        o, lse = fwd(q, k, v, causal, wl, scale)
        vis = _visible(N, causal, wl)
        for h in range(Hq):
            for i in range(N):
                np.testing.assert_allclose(o[0, h, i], v[0, 0, vis[i]].astype(np.float64).mean(axis=0),
                                           rtol=0, atol=1e-12)
                want = scale * float(q[0, h, i].astype(np.float64) @ kvec) + math.log(len(vis[i]))
                assert abs(lse[0, h, i] - want) <= 1e-12


def pin_one_hot_dominant(fwd):
    """One key's score exceeds every other visible score by at least D: O_i
    is within (n-1) e^{-D} max|V| of that key's V row."""
    N, d = 12, 3
    rng = np.random.default_rng(13)
    v = rng.standard_normal((1, 1, N, d))
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = np.arange(N)          # key j has first component j
    q = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 40.0                  # score 40*j: the largest visible j dominates
    for causal, wl in MASKS:
        o, _ = fwd(q, k, v, causal, wl, 1.0)
        vis = _visible(N, causal, wl)
        for i in range(N):
            jstar = max(vis[i])
            bound = (len(vis[i]) - 1) * math.exp(-40.0) * np.abs(v).max() * 2 + 1e-14
            assert np.abs(o[0, 0, i] - v[0, 0, jstar]).max() <= bound, (causal, wl, i)


def pin_special_cases(fwd):
    """window_left = 0 with causal: each query sees only itself, so O_i = V_i
    and lse_i = scale*<q_i, k_i>.  Causal row 0 is V_0.  N = 1 gives O = V.
    A window of N-1 or more keys with causal is plain causal."""
    B, Hq, Hkv, N, d = 2, 3, 3, 10, 5
    q, k, v = random_inputs(14, "f32", B, Hq, Hkv, N, d)
    scale = 0.45
    o, lse = fwd(q, k, v, True, 0, scale)
    np.testing.assert_allclose(o, v.astype(np.float64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scale * np.einsum("bhnd,bhnd->bhn", q.astype(np.float64),
                                                     k.astype(np.float64)), rtol=0, atol=1e-12)
    o, _ = fwd(q, k, v, True, -1, scale)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0].astype(np.float64), rtol=0, atol=1e-12)
    q1, k1, v1 = random_inputs(15, "f32", 1, 2, 1, 1, 4)
    for causal, wl in MASKS:
        o, lse = fwd(q1, k1, v1, causal, wl, scale)
        np.testing.assert_allclose(o, np.repeat(v1, 2, axis=1).astype(np.float64), rtol=0, atol=1e-12)
    oc, lc = fwd(q, k, v, True, -1, scale)
    for wl in (N - 1, N, 5 * N):
        ow, lw = fwd(q, k, v, True, wl, scale)
        np.testing.assert_allclose(ow, oc, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lw, lc, rtol=0, atol=1e-13)


def pin_key_permutation(fwd):
    """Without causal/window masks the keys form a set: permuting K and V rows
    together leaves O and lse unchanged.  A mismatched K/V row pairing fails."""
    B, Hq, Hkv, N, d = 1, 2, 2, 23, 6
    q, k, v = random_inputs(16, "f32", B, Hq, Hkv, N, d)
    perm = np.random.default_rng(17).permutation(N)
    o0, l0 = fwd(q, k, v, False, -1, 0.4)
    o1, l1 = fwd(q, k[:, :, perm], v[:, :, perm], False, -1, 0.4)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)


def pin_zero_and_negative_scale(fwd):
    """scale = 0: every visible score is 0, so O_i is the mean of the visible
    V rows and lse_i = ln(n_i).  scale < 0: torch's float64 attention agrees,
    and the keys the query is least aligned with weigh most (with q_i = k_j*
    for one key j*, that key gets the smallest probability)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 15, 6
    q, k, v = random_inputs(18, "f32", B, Hq, Hkv, N, d)
    for causal, wl in MASKS:
        o, lse = fwd(q, k, v, causal, wl, 0.0)
        vis = _visible(N, causal, wl)
        for h in range(Hq):
            for i in range(N):
                np.testing.assert_allclose(o[0, h, i], v[0, h // 2, vis[i]].astype(np.float64).mean(axis=0),
                                           rtol=0, atol=1e-12)
                assert abs(lse[0, h, i] - math.log(len(vis[i]))) <= 1e-12
        for scale in (-0.6, -1.0 / math.sqrt(d)):
            o, lse = fwd(q, k, v, causal, wl, scale)
            ro, rl = _torch_reference(q, k, v, causal, wl, scale)
            np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12, err_msg=f"o scale={scale} causal={causal} wl={wl}")
            np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12, err_msg=f"lse scale={scale}")
    # V = identity exposes P: under a negative scale the aligned key is the
    # least likely one of the row
    kk = np.random.default_rng(19).standard_normal((1, 1, 6, 6))
    qq = np.repeat(kk[:, :, 2:3], 6, axis=2) * 3.0
    P, _ = fwd(qq, kk, np.eye(6)[None, None], False, -1, -0.5)
    assert (P[0, 0].argmin(axis=-1) == 2).all()
    P, _ = fwd(qq, kk, np.eye(6)[None, None], False, -1, 0.5)
    assert (P[0, 0].argmax(axis=-1) == 2).all()


ALL_PINS = [pin_hand_worked, pin_torch_sdpa, pin_rows_are_probabilities, pin_shift_invariance,
            pin_zero_and_negative_scale,
            pin_all_equal_keys, pin_one_hot_dominant, pin_special_cases, pin_key_permutation]
