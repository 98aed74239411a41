"""Pins of the key/value-cache oracle (``oracle.attention_fwd_kvcache``).

Each pin takes the function under test, ``fn(q, k, v, seqlens, causal,
window_left, scale) -> (o, lse)``, and raises AssertionError on a mismatch.
What pins it, besides itself:

- the full forward oracle (pinned on its own against torch and closed forms):
  the cache rows are the last Nq rows of causal self-attention over the whole
  sequence, whatever the earlier rows ask -- the meaning of aligning the rows
  to the end of the cache;
- the square case Nq = Nk = L, where both alignments coincide, equals the
  forward oracle outright;
- brute force with Python loops and math.fsum on tiny inputs;
- closed forms: a row that sees one key returns that key's value row; empty
  rows give o = 0, lse = -inf; keys past a batch's length do not matter;
  grouped heads equal the same heads with K/V repeated per query head.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention_fwd
from workloads import random_inputs

TOL = 1e-12


def _case(seed, B, Hq, Hkv, Nq, Nk, d, mult=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d)) * mult
    k = rng.standard_normal((B, Hkv, Nk, d)) * mult
    v = rng.standard_normal((B, Hkv, Nk, d))
    return q, k, v


def pin_kv_last_rows_of_full_forward(fn):
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 5, 40, 8
    q, k, v = _case(900, B, Hq, Hkv, Nq, Nk, d)
    lens = [40, 23, 7]
    rng = np.random.default_rng(901)
    for causal, wl in [(True, -1), (False, -1), (True, 3), (False, 6), (True, 0)]:
        o, lse = fn(q, k, v, lens, causal, wl, 0.4)
        for b, L in enumerate(lens):
            # the whole sequence: L - Nq earlier query rows (anything), then ours
            early = rng.standard_normal((1, Hq, L - Nq, d))
            qf = np.concatenate([early, q[b:b + 1]], axis=2)
            of, lf = attention_fwd(qf, k[b:b + 1, :, :L], v[b:b + 1, :, :L], causal, wl, 0.4)
            np.testing.assert_allclose(o[b], of[0, :, L - Nq:], rtol=0, atol=TOL)
            np.testing.assert_allclose(lse[b], lf[0, :, L - Nq:], rtol=0, atol=TOL)


def pin_kv_square_equals_forward(fn):
    q, k, v = random_inputs(902, "f32", 2, 6, 3, 33, 16)
    for causal, wl in [(True, -1), (False, -1), (True, 5), (False, 0)]:
        o, lse = fn(q, k, v, None, causal, wl, 0.25)
        of, lf = attention_fwd(q, k, v, causal, wl, 0.25)
        np.testing.assert_allclose(o, of, rtol=0, atol=TOL)
        np.testing.assert_allclose(lse, lf, rtol=0, atol=TOL)


def pin_kv_brute_force(fn):
    B, Hq, Hkv, Nq, Nk, d = 2, 2, 1, 3, 6, 3
    q, k, v = _case(903, B, Hq, Hkv, Nq, Nk, d)
    lens = [6, 4]
    for causal, wl in [(True, -1), (False, -1), (True, 1), (False, 2)]:
        o, lse = fn(q, k, v, lens, causal, wl, 0.7)
        for b in range(B):
            L = lens[b]
            for h in range(Hq):
                for i in range(Nq):
                    pos = L - Nq + i
                    seen = [j for j in range(L) if (not causal or j <= pos) and (wl < 0 or j >= pos - wl)]
                    sc = {j: 0.7 * math.fsum(q[b, h, i, c] * k[b, 0, j, c] for c in range(d)) for j in seen}
                    mx = max(sc.values())
                    z = math.fsum(math.exp(s - mx) for s in sc.values())
                    assert abs(lse[b, h, i] - (mx + math.log(z))) <= TOL
                    for c in range(d):
                        ref = math.fsum(math.exp(sc[j] - mx) / z * v[b, 0, j, c] for j in seen)
                        assert abs(o[b, h, i, c] - ref) <= TOL


def pin_kv_empty_rows(fn):
    q, k, v = _case(904, 2, 2, 2, 6, 10, 4)
    o, lse = fn(q, k, v, [4, 0], True, -1, 0.5)
    # batch 0: positions -2, -1 see nothing; rows 2.. see keys 0..i-2
    assert (o[0, :, :2] == 0).all() and np.isneginf(lse[0, :, :2]).all()
    assert np.isfinite(lse[0, :, 2:]).all()
    np.testing.assert_allclose(o[0, :, 2], v[0, :, 0], rtol=0, atol=TOL)   # only key 0
    # batch 1: an empty cache
    assert (o[1] == 0).all() and np.isneginf(lse[1]).all()
    # without a causal mask an empty cache is still empty, a non-empty one is not
    o2, l2 = fn(q, k, v, [4, 0], False, -1, 0.5)
    assert np.isfinite(l2[0]).all() and np.isneginf(l2[1]).all() and (o2[1] == 0).all()


def pin_kv_single_key(fn):
    q, k, v = _case(905, 2, 3, 3, 4, 12, 5)
    lens = [12, 9]
    o, lse = fn(q, k, v, lens, True, 0, 0.3)
    for b, L in enumerate(lens):
        for i in range(4):
            pos = L - 4 + i
            np.testing.assert_allclose(o[b, :, i], v[b, :, pos], rtol=0, atol=TOL)
            s = 0.3 * np.einsum("hc,hc->h", q[b, :, i], k[b, :, pos])
            np.testing.assert_allclose(lse[b, :, i], s, rtol=0, atol=TOL)


def pin_kv_tail_is_ignored(fn):
    q, k, v = _case(906, 2, 4, 2, 3, 20, 6)
    lens = [11, 17]
    o, lse = fn(q, k, v, lens, False, -1, 0.5)
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(lens):
        k2[b, :, L:] = 1e6
        v2[b, :, L:] = -1e6
    o2, l2 = fn(q, k2, v2, lens, False, -1, 0.5)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def pin_kv_gqa_equals_repeated_heads(fn):
    G = 3
    q, k, v = _case(907, 2, 2 * G, 2, 4, 15, 5)
    lens = [15, 8]
    o, lse = fn(q, k, v, lens, True, 4, 0.6)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o2, l2 = fn(q, kr, vr, lens, True, 4, 0.6)
    np.testing.assert_allclose(o, o2, rtol=0, atol=TOL)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=TOL)


ALL_KV_PINS = [pin_kv_last_rows_of_full_forward, pin_kv_square_equals_forward, pin_kv_brute_force,
               pin_kv_empty_rows, pin_kv_single_key, pin_kv_tail_is_ignored, pin_kv_gqa_equals_repeated_heads]
