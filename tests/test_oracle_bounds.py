"""CPU tests of the oracles' error-bound magnitudes (no GPU): the pins of
``tests/oracle_bound_pins.py`` on the oracles, and planted mistakes in the
magnitude code, each of which must fail at least one of those pins."""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

from oracle import attention_bwd, attention_bwd_varlen, attention_fwd
from tests import oracle_bound_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def fwd_mag(q, k, v, causal, wl, scale, frac):
    return attention_fwd(q, k, v, causal, wl, scale, threads=1, tail=frac)


def bwd_mag(q, k, v, do, causal, wl, scale):
    return attention_bwd(q, k, v, do, causal, wl, scale, threads=1, bounds=True)


def bwd_varlen_mag(q, k, v, do, cq, ck, **kw):
    return attention_bwd_varlen(q, k, v, do, cq, ck, threads=1, bounds=True, **kw)


@pytest.mark.parametrize("pin", pins.FWD_MAG_PINS, ids=lambda p: p.__name__)
def test_fwd_magnitude_pin(pin):
    pin(fwd_mag)


@pytest.mark.parametrize("pin", pins.BWD_MAG_PINS, ids=lambda p: p.__name__)
def test_bwd_magnitude_pin(pin):
    pin(bwd_mag)


@pytest.mark.parametrize("pin", pins.VARLEN_BWD_MAG_PINS, ids=lambda p: p.__name__)
def test_varlen_bwd_magnitude_pin(pin):
    pin(bwd_varlen_mag)


def _load_mutant(fname, old, new, modname):
    path = os.path.join(ROOT, "oracle", fname)
    src = open(path).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType(f"oracle.{modname}")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), modname, "exec"), mod.__dict__)
    return mod


def _caught(pin_list, fn):
    caught = []
    for pin in pin_list:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    return caught


FWD_MAG_MUTANTS = [
    ("P|V| from the unnormalised exponentials", "mag_pv[s0:s0 + len(r)] = P @ np.abs(vh)",
     "mag_pv[s0:s0 + len(r)] = E @ np.abs(vh)"),
    ("P|V| without the absolute value", "mag_pv[s0:s0 + len(r)] = P @ np.abs(vh)",
     "mag_pv[s0:s0 + len(r)] = P @ vh"),
    ("tail threshold absolute, not relative to the row max",
     "np.minimum(P, tail * P.max(axis=1, keepdims=True))", "np.minimum(P, tail)"),
    ("tail threshold relative to the column max",
     "np.minimum(P, tail * P.max(axis=1, keepdims=True))", "np.minimum(P, tail * P.max(axis=0, keepdims=True))"),
    ("tail weighted by |K| instead of |V|", "mag_tail[s0:s0 + len(r)] = small @ np.abs(vh)",
     "mag_tail[s0:s0 + len(r)] = small @ np.abs(kh)"),
    ("score magnitude without |Q|", "A = abs(scale) * (np.abs(qh[r]) @ np.abs(kh).T)", "A = abs(scale) * (qh[r] @ np.abs(kh).T)"),
    ("score magnitude without the scale", "A = abs(scale) * (np.abs(qh[r]) @ np.abs(kh).T)",
     "A = (np.abs(qh[r]) @ np.abs(kh).T)"),
    ("score magnitude with the signed scale", "A = abs(scale) * (np.abs(qh[r]) @ np.abs(kh).T)",
     "A = scale * (np.abs(qh[r]) @ np.abs(kh).T)"),
    ("score magnitude over masked keys too", "            A[masked(r[:, None], keys[None, :], causal, window_left)] = 0.0\n",
     ""),
]


@pytest.mark.parametrize("name,old,new", FWD_MAG_MUTANTS, ids=[m[0] for m in FWD_MAG_MUTANTS])
def test_fwd_magnitude_pins_catch_planted_mistake(name, old, new):
    mod = _load_mutant("attention_ref.py", old, new, "ref_mag_mutant")
    fn = lambda q, k, v, c, w, s, f: mod.attention_fwd(q, k, v, c, w, s, threads=1, tail=f)  # noqa: E731
    assert _caught(pins.FWD_MAG_PINS, fn), f"no pin caught the planted mistake: {name}"


BWD_MAG_MUTANTS = [
    ("dq without the scale", 'mag["dq"][g, r] = abs(scale) * (A @ np.abs(kh))', 'mag["dq"][g, r] = (A @ np.abs(kh))'),
    ("dq with the scale twice", 'mag["dq"][g, r] = abs(scale) * (A @ np.abs(kh))',
     'mag["dq"][g, r] = scale * scale * (A @ np.abs(kh))'),
    ("dq through |Q| instead of |K|", 'mag["dq"][g, r] = abs(scale) * (A @ np.abs(kh))',
     'mag["dq"][g, r] = scale * (A @ np.abs(qh[r]))'),
    ("dq through |V| instead of |K|", 'mag["dq"][g, r] = abs(scale) * (A @ np.abs(kh))',
     'mag["dq"][g, r] = scale * (A @ np.abs(vh))'),
    ("dq with the signed scale", 'mag["dq"][g, r] = abs(scale) * (A @ np.abs(kh))',
     'mag["dq"][g, r] = scale * (A @ np.abs(kh))'),
    ("dk through |K| instead of |Q|", 'mag["dk"] += abs(scale) * (A.T @ np.abs(qh[r]))',
     'mag["dk"] += abs(scale) * (A.T @ np.abs(kh))'),
    ("dk without the scale", 'mag["dk"] += abs(scale) * (A.T @ np.abs(qh[r]))', 'mag["dk"] += (A.T @ np.abs(qh[r]))'),
    ("dk with the signed scale", 'mag["dk"] += abs(scale) * (A.T @ np.abs(qh[r]))',
     'mag["dk"] += scale * (A.T @ np.abs(qh[r]))'),
    ("dk not summed over the group", 'mag["dk"] += abs(scale) * (A.T @ np.abs(qh[r]))',
     'mag["dk"] = abs(scale) * (A.T @ np.abs(qh[r]))'),
    ("|dS| replaced by dS", "A = np.abs(dS)", "A = dS"),
    ("|dS| replaced by |dP|", "A = np.abs(dS)", "A = np.abs(dP)"),
    ("dv from the unnormalised exponentials", 'mag["dv"] += P.T @ np.abs(doh[r])', 'mag["dv"] += E.T @ np.abs(doh[r])'),
    ("dv without the absolute value", 'mag["dv"] += P.T @ np.abs(doh[r])', 'mag["dv"] += P.T @ doh[r]'),
    ("row term without |dO|", "F = (np.abs(doh[r]) * (P @ np.abs(vh)))", "F = (doh[r] * (P @ np.abs(vh)))"),
    ("row term from O instead of P|V|", "F = (np.abs(doh[r]) * (P @ np.abs(vh)))", "F = (np.abs(doh[r]) * (P @ vh))"),
    ("dq_f without P", "PF = P * F", "PF = F + 0 * P"),
    ("dq_f without the scale", 'mag["dq_f"][g, r] = abs(scale) * (PF @ np.abs(kh))',
     'mag["dq_f"][g, r] = (PF @ np.abs(kh))'),
    ("dq_f with the signed scale", 'mag["dq_f"][g, r] = abs(scale) * (PF @ np.abs(kh))',
     'mag["dq_f"][g, r] = scale * (PF @ np.abs(kh))'),
    ("dk_f through |K| instead of |Q|", 'mag["dk_f"] += abs(scale) * (PF.T @ np.abs(qh[r]))',
     'mag["dk_f"] += abs(scale) * (PF.T @ np.abs(kh))'),
    ("visibility from the masked set", "Vis = (~hidden).astype(np.float64)", "Vis = hidden.astype(np.float64)"),
    ("visibility weighted by P", "Vis = (~hidden).astype(np.float64)", "Vis = (~hidden) * P"),
    ("dv_v through |Q|", 'mag["dv_v"] += Vis.T @ np.abs(doh[r])', 'mag["dv_v"] += Vis.T @ np.abs(qh[r])'),
    ("dq_v without the scale", 'mag["dq_v"][g, r] = abs(scale) * (Vis @ np.abs(kh))',
     'mag["dq_v"][g, r] = (Vis @ np.abs(kh))'),
    ("dk_v not summed over the group", 'mag["dk_v"] += abs(scale) * (Vis.T @ np.abs(qh[r]))',
     'mag["dk_v"] = abs(scale) * (Vis.T @ np.abs(qh[r]))'),
    ("dk_f not summed over the group", 'mag["dk_f"] += abs(scale) * (PF.T @ np.abs(qh[r]))',
     'mag["dk_f"] = abs(scale) * (PF.T @ np.abs(qh[r]))'),
]


@pytest.mark.parametrize("name,old,new", BWD_MAG_MUTANTS, ids=[m[0] for m in BWD_MAG_MUTANTS])
def test_bwd_magnitude_pins_catch_planted_mistake(name, old, new):
    mod = _load_mutant("attention_bwd_ref.py", old, new, "bwd_mag_mutant")
    fn = lambda q, k, v, do, c, w, s: mod.attention_bwd(q, k, v, do, c, w, s, threads=1, bounds=True)  # noqa: E731
    assert _caught(pins.BWD_MAG_PINS, fn), f"no pin caught the planted mistake: {name}"


VARLEN_MAG_MUTANTS = [
    ("packed dq magnitude not scattered back", 'mags["dq"][q0:q1, h] = mag["dq"][gi]',
     'mags["dq"][q0:q1, h] = 0 * mag["dq"][gi]'),
    ("packed dk_f magnitude not scattered back", 'mags["dk_f"][k0:k1, hk] = mag["dk_f"]',
     'mags["dk_f"][k0:k1, hk] = 0 * mag["dk_f"]'),
    ("packed magnitudes with queries at the start of the keys", "pos = r + shift", "pos = r"),
]


@pytest.mark.parametrize("name,old,new", VARLEN_MAG_MUTANTS, ids=[m[0] for m in VARLEN_MAG_MUTANTS])
def test_varlen_magnitude_pins_catch_planted_mistake(name, old, new):
    mod = _load_mutant("attention_bwd_ref.py", old, new, "bwd_varlen_mag_mutant")
    fn = lambda *a, **kw: mod.attention_bwd_varlen(*a, threads=1, bounds=True, **kw)  # noqa: E731
    assert _caught(pins.VARLEN_BWD_MAG_PINS, fn), f"no pin caught the planted mistake: {name}"
