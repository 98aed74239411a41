"""CPU tests of the gradient oracle (no GPU): every pin, the magnitude terms
used for error bounds, and planted mistakes that the pins must catch."""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

from oracle import attention_bwd, attention_bwd_varlen
from tests import oracle_bwd_pins as pins
from workloads import random_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ref_bwd(q, k, v, do, causal, wl, scale):
    return attention_bwd(q, k, v, do, causal, wl, scale)


@pytest.mark.parametrize("pin", pins.ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pin(pin):
    pin(ref_bwd)


def test_bwd_threads_and_row_blocks_agree():
    """More rows than one block, several worker threads: same numbers as one
    thread (each worker owns whole key/value heads)."""
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 8
    q, k, v = random_inputs(800, "f32", B, Hq, Hkv, N, d)
    do = np.random.default_rng(801).standard_normal((B, Hq, N, d))
    a = attention_bwd(q, k, v, do, True, 40, 0.3, threads=1)
    b = attention_bwd(q, k, v, do, True, 40, 0.3, threads=4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bwd_magnitudes_bound_the_gradients():
    """The absolute-value products dominate the gradients they bound."""
    B, Hq, Hkv, N, d = 1, 4, 2, 40, 8
    q, k, v = random_inputs(810, "f32", B, Hq, Hkv, N, d)
    do = np.random.default_rng(811).standard_normal((B, Hq, N, d))
    dq, dk, dv, mag = attention_bwd(q, k, v, do, True, 7, 0.5, bounds=True)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert (np.abs(g) <= mag[name] * (1 + 1e-12) + 1e-15).all(), name
        assert mag[name].max() > 0
    assert (mag["dq_f"] >= 0).all() and (mag["dk_f"] >= 0).all()
    g2 = attention_bwd(q, k, v, do, True, 7, 0.5)
    for x, y in zip((dq, dk, dv), g2):
        np.testing.assert_array_equal(x, y)


def test_bwd_rejects_bad_arguments():
    q, k, v = random_inputs(820, "f32", 1, 3, 2, 4, 4)
    do = np.zeros_like(q)
    with pytest.raises(ValueError):
        attention_bwd(q, k, v, do)
    q, k, v = random_inputs(821, "f32", 1, 2, 1, 4, 4)
    with pytest.raises(ValueError):
        attention_bwd(q, k, v, np.zeros((1, 2, 4, 3)))
    with pytest.raises(ValueError):
        attention_bwd(q, k, v, np.zeros_like(q), window_left=-2)


def test_bwd_empty():
    q, k, v = random_inputs(830, "f32", 1, 2, 1, 0, 4)
    dq, dk, dv = attention_bwd(q, k, v, np.zeros_like(q))
    assert dq.shape == (1, 2, 0, 4) and dk.shape == (1, 1, 0, 4) and dv.shape == (1, 1, 0, 4)


# ---------------------------------------------------------------------------
# Planted mistakes: each edit of the gradient oracle's source must fail at
# least one pin.

BWD_MUTANTS = [
    ("softmax Jacobian without the row term", "dS = P * (dP - rowdot)", "dS = P * dP"),
    ("softmax Jacobian with the wrong sign", "dS = P * (dP - rowdot)", "dS = P * (rowdot - dP)"),
    ("row term without P", "rowdot = (P * dP).sum(axis=1, keepdims=True)", "rowdot = dP.sum(axis=1, keepdims=True)"),
    ("dK without the scale", "dk += scale * (dS.T @ qh[r])", "dk += (dS.T @ qh[r])"),
    ("dQ without the scale", "dq[g, r] = scale * (dS @ kh)", "dq[g, r] = (dS @ kh)"),
    ("dQ through V", "dq[g, r] = scale * (dS @ kh)", "dq[g, r] = scale * (dS @ vh)"),
    ("dK through dO", "dk += scale * (dS.T @ qh[r])", "dk += scale * (dS.T @ doh[r])"),
    ("dP through K", "dP = doh[r] @ vh.T", "dP = doh[r] @ kh.T"),
    ("dV through Q", "dv += P.T @ doh[r]", "dv += P.T @ qh[r]"),
    ("dV from scores, not probabilities", "dv += P.T @ doh[r]", "dv += E.T @ doh[r]"),
    ("group sum dropped for dK", "dk += scale * (dS.T @ qh[r])", "dk = scale * (dS.T @ qh[r])"),
    ("mask ignored in the backward", "S[hidden] = -np.inf", "S[hidden] = S[hidden]"),
    ("scores without the scale", "S = scale * (qh[r] @ kh.T)", "S = (qh[r] @ kh.T)"),
]


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_pins_catch_planted_mistake(name, old, new):
    path = os.path.join(ROOT, "oracle", "attention_bwd_ref.py")
    src = open(path).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.bwd_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "bwd_mutant", "exec"), mod.__dict__)
    bwd = lambda q, k, v, do, c, w, s: mod.attention_bwd(q, k, v, do, c, w, s, threads=1)  # noqa: E731
    caught = []
    for pin in pins.ALL_BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bwd)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


# ---------------------------------------------------------------------------
# Packed sequences of different lengths

VARLEN_MUTANTS = [
    ("queries aligned to the start of the keys", "pos = r + shift", "pos = r"),
    ("rows that see no key divide by zero", "P = E / np.where(z > 0, z, 1.0)", "P = E / z"),
    ("rows that see no key keep their max", "m[~np.isfinite(m)] = 0.0", "pass"),
    ("dK of a sequence not scattered back", "dk[k0:k1, hk] = gk", "dk[k0:k1, hk] = 0 * gk"),
]


@pytest.mark.parametrize("pin", pins.ALL_VARLEN_BWD_PINS, ids=lambda f: f.__name__)
def test_varlen_bwd_oracle_pin(pin):
    pin(lambda *a, **kw: attention_bwd_varlen(*a, threads=1, **kw))


def test_varlen_bwd_rejects_bad_arguments():
    q = np.zeros((5, 2, 4))
    k = np.zeros((7, 1, 4))
    with pytest.raises(ValueError):
        attention_bwd_varlen(q, k, k, q, [0, 2, 4], [0, 3, 7])  # q offsets stop short
    with pytest.raises(ValueError):
        attention_bwd_varlen(q, k, k, q, [0, 3, 5], [0, 4, 3, 7])
    with pytest.raises(ValueError):
        attention_bwd_varlen(q, k, k, q, [0, 3, 5], [0, 3, 7], window_left=-2)


@pytest.mark.parametrize("name,old,new", VARLEN_MUTANTS, ids=[m[0] for m in VARLEN_MUTANTS])
def test_varlen_bwd_pins_catch_planted_mistake(name, old, new):
    path = os.path.join(ROOT, "oracle", "attention_bwd_ref.py")
    src = open(path).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.bwd_varlen_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "bwd_varlen_mutant", "exec"), mod.__dict__)
    bwd = lambda *a, **kw: mod.attention_bwd_varlen(*a, threads=1, **kw)  # noqa: E731
    caught = []
    for pin in pins.ALL_VARLEN_BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bwd)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
