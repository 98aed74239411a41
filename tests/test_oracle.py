"""CPU tests of the oracle (no GPU): every pin on each oracle form, plus
planted-mistake checks that show the pins would catch the usual slips."""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention_fwd, attention_online, attention_twopass
from tests import oracle_pins as pins
from workloads import random_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ref_fwd(q, k, v, causal, wl, scale):
    return attention_fwd(q, k, v, causal, wl, scale)


def twopass_fwd(q, k, v, causal, wl, scale):
    o, lse = attention_twopass(np.asarray(q, np.float64).tolist(), np.asarray(k, np.float64).tolist(),
                               np.asarray(v, np.float64).tolist(), causal, wl, scale)
    return np.array(o, dtype=np.float64), np.array(lse, dtype=np.float64)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ref_fwd)


@pytest.mark.parametrize("Br,Bc", [(64, 64), (3, 5), (7, 2), (16, 1), (1, 16)])
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_online_emulation_pin(pin, Br, Bc):
    pin(lambda q, k, v, c, w, s: attention_online(q, k, v, c, w, s, Br=Br, Bc=Bc))


@pytest.mark.parametrize("pin", [pins.pin_hand_worked, pins.pin_rows_are_probabilities,
                                 pins.pin_all_equal_keys, pins.pin_one_hot_dominant,
                                 pins.pin_special_cases, pins.pin_key_permutation],
                         ids=lambda p: p.__name__)
def test_twopass_pin(pin):
    pin(twopass_fwd)


@pytest.mark.parametrize("causal,wl", pins.MASKS)
def test_three_forms_agree(causal, wl):
    """Brute force (loops), vectorised standard attention, and the tiled online
    form agree to 1e-12 on tiny shapes, with GQA and ragged blocks."""
    q, k, v = random_inputs(21, "bf16", 2, 4, 2, 11, 8)
    o0, l0 = attention_fwd(q, k, v, causal, wl, 0.3)
    o1, l1 = twopass_fwd(q, k, v, causal, wl, 0.3)
    o2, l2 = attention_online(q, k, v, causal, wl, 0.3, Br=4, Bc=3)
    o3, l3 = attention_online(q, k, v, causal, wl, 0.3, Br=5, Bc=4, skip_masked_blocks=False)
    for o, l in ((o1, l1), (o2, l2), (o3, l3)):
        np.testing.assert_allclose(o, o0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l0, rtol=0, atol=1e-12)


def test_rows_subset_matches_full():
    q, k, v = random_inputs(22, "f16", 1, 2, 1, 300, 16)
    rows = [0, 1, 17, 255, 256, 299]
    of, lf = attention_fwd(q, k, v, True, 40, 0.25)
    os_, ls = attention_fwd(q, k, v, True, 40, 0.25, rows=rows)
    np.testing.assert_array_equal(os_, of[:, :, rows])
    np.testing.assert_array_equal(ls, lf[:, :, rows])


def test_oracle_rejects_bad_arguments():
    q, k, v = random_inputs(23, "f32", 1, 3, 2, 4, 4)
    with pytest.raises(ValueError):
        attention_fwd(q, k, v)          # 3 query heads over 2 KV heads
    q, k, v = random_inputs(23, "f32", 1, 2, 2, 4, 4)
    with pytest.raises(ValueError):
        attention_fwd(q, k, v, window_left=-2)


# ---------------------------------------------------------------------------
# Planted mistakes: each edit of the oracle's source must fail at least one pin.

MUTANTS = [
    ("swapped Q and K in the score product", "S = scale * (qh[r] @ kh.T)", "S = scale * (kh[r] @ qh.T)"),
    ("dropped scale", "S = scale * (qh[r] @ kh.T)", "S = (qh[r] @ kh.T)"),
    ("causal hides the diagonal", "m |= j > i", "m |= j >= i"),
    ("causal hides the past", "m |= j > i", "m |= j < i"),
    ("window one key short", "m |= j < i - window_left", "m |= j <= i - window_left"),
    ("window one key long", "m |= j < i - window_left", "m |= j < i - window_left - 1"),
    ("strided GQA grouping", "return h // (Hq // Hkv)", "return h % Hkv"),
    ("lse in base 2", "m[:, 0] + np.log(z[:, 0])", "m[:, 0] + np.log2(z[:, 0])"),
    ("lse without the max", "m[:, 0] + np.log(z[:, 0])", "np.log(z[:, 0])"),
    ("missing normalisation", "P = E / z", "P = E"),
    ("wrong sign of max shift", "E = np.exp(S - m)", "E = np.exp(S + m)"),
    ("K used as V", "= P @ vh", "= P @ kh"),
    ("masked scores zeroed instead of -inf", "window_left)] = -np.inf", "window_left)] = 0.0"),
    ("mask ignored", "window_left)] = -np.inf", "window_left)] = S[masked(r[:, None], keys[None, :], causal, window_left)]"),
]


def _mutant_fwd(src_old, src_new):
    path = os.path.join(ROOT, "oracle", "attention_ref.py")
    src = open(path).read()
    assert src_old in src, f"mutation anchor not found: {src_old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src.replace(src_old, src_new), "oracle_mutant", "exec"), mod.__dict__)
    return lambda q, k, v, c, w, s: mod.attention_fwd(q, k, v, c, w, s, threads=1)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    fwd = _mutant_fwd(old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fwd)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


ONLINE_MUTANTS = [
    ("no rescale of the partial output", "acc = alpha[:, None] * acc + P @ v", "acc = acc + P @ v"),
    ("no rescale of the running sum", "l = alpha * l + P.sum(axis=1)", "l = l + P.sum(axis=1)"),
    ("running max never updated", "m = m_new", "m = m"),
]


@pytest.mark.parametrize("name,old,new", ONLINE_MUTANTS, ids=[m[0] for m in ONLINE_MUTANTS])
def test_pins_catch_planted_online_mistake(name, old, new):
    path = os.path.join(ROOT, "oracle", "online_emul.py")
    src = open(path).read()
    assert old in src
    mod = types.ModuleType("oracle.online_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "online_mutant", "exec"), mod.__dict__)
    fwd = lambda q, k, v, c, w, s: mod.attention_online(q, k, v, c, w, s, Br=4, Bc=3)  # noqa: E731
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fwd)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


def test_oracle_is_independent_of_gpu_path():
    """The oracle imports nothing from the GPU package, and the package and
    the bench's timed path import nothing from the oracle."""
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith(".py"):
            src = open(os.path.join(ROOT, "oracle", fn)).read()
            assert "exact_tiled_attention_04_amd" not in src, fn
    pkg = os.path.join(ROOT, "exact_tiled_attention_04_amd")
    if os.path.isdir(pkg):
        for dirpath, _, files in os.walk(pkg):
            for fn in files:
                if fn.endswith((".py", ".cpp", ".hip", ".h")):
                    src = open(os.path.join(dirpath, fn)).read()
                    assert "import oracle" not in src and "from oracle" not in src, fn
    assert oracle.attention_fwd is attention_fwd


def test_magnitudes_bound_the_output_and_leave_it_unchanged():
    """The optional magnitudes: P|V| dominates |O|, the tail term lies
    between 0 and P|V| and grows with the fraction, O and lse are unchanged."""
    q, k, v = random_inputs(850, "f32", 1, 4, 2, 90, 16, mult=2.0)
    o, lse = attention_fwd(q, k, v, True, 30, 0.4)
    o2, lse2, m1 = attention_fwd(q, k, v, True, 30, 0.4, tail=2 ** -10)
    _, _, m2 = attention_fwd(q, k, v, True, 30, 0.4, tail=2 ** -4)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    assert (np.abs(o) <= m1["pv"] * (1 + 1e-12)).all()
    assert (m1["tail"] >= 0).all() and (m1["tail"] <= m1["pv"] * (1 + 1e-12)).all()
    assert (m2["tail"] >= m1["tail"] - 1e-15).all() and m2["tail"].max() > m1["tail"].max()
    # a zero fraction leaves no tail
    _, _, m0 = attention_fwd(q, k, v, True, 30, 0.4, tail=0.0)
    np.testing.assert_array_equal(m0["tail"], 0.0)
    # sabs bounds every visible score, and is the largest one for
    # nonnegative inputs (brute force over the visible keys)
    qa, ka, va = np.abs(q).astype(np.float64), np.abs(k).astype(np.float64), v
    _, _, ma = attention_fwd(qa, ka, va, True, 30, 0.4, tail=0.0)
    for b, h, i in [(0, 0, 0), (0, 1, 45), (0, 3, 89), (0, 2, 31)]:
        hk = h // 2
        js = [j for j in range(90) if j <= i and j >= i - 30]
        s_pos = max(0.4 * float(qa[b, h, i] @ ka[b, hk, j]) for j in js)
        assert abs(ma["sabs"][b, h, i] - s_pos) <= 1e-12 * s_pos
        s_abs = max(abs(0.4 * float(q[b, h, i].astype(np.float64) @ k[b, hk, j])) for j in js)
        assert m1["sabs"][b, h, i] >= s_abs
