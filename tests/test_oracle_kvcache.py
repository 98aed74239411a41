"""CPU tests of the key/value-cache oracle (no GPU): every pin, and planted
mistakes that the pins must catch."""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

from oracle import attention_fwd_kvcache
from tests import oracle_kvcache_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ref(q, k, v, lens, causal, wl, scale):
    return attention_fwd_kvcache(q, k, v, lens, causal, wl, scale)


@pytest.mark.parametrize("pin", pins.ALL_KV_PINS, ids=lambda p: p.__name__)
def test_kv_oracle_pin(pin):
    pin(ref)


def test_kv_threads_agree():
    rng = np.random.default_rng(910)
    q = rng.standard_normal((3, 8, 4, 16))
    k = rng.standard_normal((3, 2, 50, 16))
    v = rng.standard_normal((3, 2, 50, 16))
    a = attention_fwd_kvcache(q, k, v, [50, 3, 20], True, 9, 0.2, threads=1)
    b = attention_fwd_kvcache(q, k, v, [50, 3, 20], True, 9, 0.2, threads=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_kv_rejects_bad_arguments():
    q, k, v = np.zeros((1, 3, 2, 4)), np.zeros((1, 2, 5, 4)), np.zeros((1, 2, 5, 4))
    with pytest.raises(ValueError):
        attention_fwd_kvcache(q, k, v)
    q = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        attention_fwd_kvcache(q, k, v, [6])
    with pytest.raises(ValueError):
        attention_fwd_kvcache(q, k, v, [-1])
    with pytest.raises(ValueError):
        attention_fwd_kvcache(q, k, v, None, window_left=-2)
    with pytest.raises(ValueError):
        attention_fwd_kvcache(q, k, v[:, :, :, :3])


KV_MUTANTS = [
    ("rows aligned to the start of the cache", "p = (L - Nq + np.arange(Nq))[:, None]", "p = (np.arange(Nq))[:, None]"),
    ("causal mask hides the row's own key", "vis &= j <= p", "vis &= j < p"),
    ("window one key short", "vis &= j >= p - window_left", "vis &= j > p - window_left"),
    ("lengths ignored", "kh = k[b, hk, :L].astype(np.float64)", "kh = k[b, hk].astype(np.float64)"),
    ("empty rows not special-cased", "rows = vis.any(axis=1)", "rows = np.ones(Nq, dtype=bool)"),
    ("strided head grouping", "hk = kv_head_of(h, Hq, Hkv)", "hk = h % Hkv"),
    ("scores without the scale", "S = scale * (q[b, h].astype(np.float64) @ kh.T)",
     "S = (q[b, h].astype(np.float64) @ kh.T)"),
    ("lse without the max", "lse[b, h, rows] = m[:, 0] + np.log(z[:, 0])", "lse[b, h, rows] = np.log(z[:, 0])"),
]


@pytest.mark.parametrize("name,old,new", KV_MUTANTS, ids=[m[0] for m in KV_MUTANTS])
def test_kv_pins_catch_planted_mistake(name, old, new):
    path = os.path.join(ROOT, "oracle", "attention_kvcache_ref.py")
    src = open(path).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.kv_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "kv_mutant", "exec"), mod.__dict__)
    fn = lambda q, k, v, lens, c, w, s: mod.attention_fwd_kvcache(q, k, v, lens, c, w, s, threads=1)  # noqa: E731
    caught = []
    for pin in pins.ALL_KV_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


# --- packed variable-length form ---------------------------------------------

from oracle import attention_fwd, attention_fwd_varlen  # noqa: E402


def _pack(x):
    """[B, H, N, d] -> [B*N, H, d] (sequence-major packing)."""
    B, H, N, d = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B * N, H, d))


def test_varlen_equal_lengths_equal_the_batched_forward():
    """Packed sequences of one length give the batched forward oracle's
    result (pinned on its own against torch)."""
    rng = np.random.default_rng(920)
    B, Hq, Hkv, N, d = 3, 4, 2, 37, 8
    q, k, v = (rng.standard_normal(s) for s in [(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)])
    cu = np.arange(B + 1) * N
    for causal, wl in [(True, -1), (False, -1), (True, 5), (False, 3)]:
        o, lse = attention_fwd_varlen(_pack(q), _pack(k), _pack(v), cu, cu, causal, wl, 0.3)
        of, lf = attention_fwd(q, k, v, causal, wl, 0.3)
        np.testing.assert_allclose(o, _pack(of), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lf.transpose(1, 0, 2).reshape(Hq, B * N), rtol=0, atol=1e-12)


def test_varlen_sequences_are_independent():
    """Each packed sequence equals the forward oracle run on it alone (square
    sequences), and a sequence with fewer queries than keys equals the last
    rows of the forward over its keys; empty sequences contribute nothing."""
    rng = np.random.default_rng(921)
    Hq, Hkv, d = 4, 2, 8
    lq = [5, 0, 12, 7, 1]
    lk = [5, 0, 12, 19, 30]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((cq[-1], Hq, d))
    k = rng.standard_normal((ck[-1], Hkv, d))
    v = rng.standard_normal((ck[-1], Hkv, d))
    o, lse = attention_fwd_varlen(q, k, v, cq, ck, True, -1, 0.5)
    for b in range(5):
        if lq[b] == 0:
            continue
        L = lk[b]
        early = rng.standard_normal((1, Hq, L - lq[b], d))
        qf = np.concatenate([early, q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]], axis=2)
        of, lf = attention_fwd(qf, k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None],
                               v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None], True, -1, 0.5)
        np.testing.assert_allclose(o[cq[b]:cq[b + 1]], of[0, :, L - lq[b]:].transpose(1, 0, 2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, cq[b]:cq[b + 1]], lf[0, :, L - lq[b]:], rtol=0, atol=1e-12)


def test_varlen_more_queries_than_keys_and_bad_offsets():
    rng = np.random.default_rng(922)
    q = rng.standard_normal((6, 2, 4))
    k = rng.standard_normal((2, 1, 4))
    v = rng.standard_normal((2, 1, 4))
    o, lse = attention_fwd_varlen(q, k, v, [0, 6], [0, 2], True, -1, 1.0)
    assert (o[:4] == 0).all() and np.isneginf(lse[:, :4]).all()   # positions -4 .. -1 see nothing
    np.testing.assert_allclose(o[4], np.repeat(v[0], 2, axis=0), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        attention_fwd_varlen(q, k, v, [0, 5], [0, 2])
    with pytest.raises(ValueError):
        attention_fwd_varlen(q, k, v, [0, 4, 6], [0, 3, 2])
