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
