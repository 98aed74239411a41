"""Pins for the oracles' error-bound magnitudes, from above as well as below.

The forward oracle's optional magnitudes (``attention_fwd(..., tail=f)``:
'pv' = P|V|, 'tail' = sum_j min(p_ij, f max_j p_ij) |v_j|, 'sabs') and the
gradient oracle's (``attention_bwd(..., bounds=True)``: 'dv' = P^T |dO|,
'dq' = |scale| |dS| |K|, 'dk' = |scale| |dS|^T |Q|, 'dq_f', 'dk_f' from the row
terms F_i = sum_c |do_ic| (P|V|)_ic) set how wide the parity bounds of the
backward and FP8 kernels are.  Checking only that they dominate |O| or |g|
would let a bound that is too loose (probabilities left unnormalised, a
doubled scale, the wrong operand's absolute values) pass unnoticed, so each
term is pinned to its value:

- closed forms: V >= 0 makes P|V| equal to O; a fraction f >= 1 makes the
  tail equal to P|V|; equal keys make every visible probability 1/n_i, so the
  tail is f P|V|; dO >= 0 makes P^T|dO| equal to dV; for dO, V >= 0 the row
  term F_i is sum_c do_ic o_ic, and with K (or Q) all ones the F products
  reduce to scale F_i (or sums of p_ij F_i); a row that sees exactly two keys
  has |dS_i0| = |dS_i1| = p_i0 p_i1 |dP_i0 - dP_i1| with p_i0 the logistic
  function of s_i0 - s_i1;
- brute force: every term recomputed element by element with Python loops,
  ``math.exp`` and ``math.fsum`` on tiny inputs, all mask kinds, GQA, positive,
  negative and zero scales (the terms are magnitudes: they carry |scale|).

Each pin takes the oracle callable and raises AssertionError on a mismatch;
``tests/test_oracle_bounds.py`` runs them on the oracle and on copies of it
with planted mistakes, each of which must fail at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

from workloads import random_inputs

MASKS = [(False, -1), (True, -1), (False, 0), (False, 3), (True, 0), (True, 2), (True, 5)]


def _hidden(pos, j, causal, wl):
    return (causal and j > pos) or (wl >= 0 and j < pos - wl)


# ---------------------------------------------------------------------------
# Brute force: one query row at a time, scalar loops, exact summation.

def _row_probs(qi, kh, pos, causal, wl, scale):
    """Scores and probabilities of one query row (at key position ``pos``)
    by loops: returns (list of visible j, {j: p_ij}, {j: s_ij})."""
    Nk, d = kh.shape
    vis = [j for j in range(Nk) if not _hidden(pos, j, causal, wl)]
    s = {j: scale * math.fsum(float(qi[c]) * float(kh[j, c]) for c in range(d)) for j in vis}
    if not vis:
        return vis, {}, s
    m = max(s.values())
    e = {j: math.exp(s[j] - m) for j in vis}
    z = math.fsum(e.values())
    return vis, {j: e[j] / z for j in vis}, s


def fwd_mags_brute(q, k, v, causal, wl, scale, frac):
    """'pv', 'tail', 'sabs' of the forward, element by element."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    pv = np.zeros((B, Hq, N, d))
    tail = np.zeros((B, Hq, N, d))
    sabs = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kh, vh = k[b, h // g], v[b, h // g]
            for i in range(N):
                vis, p, _ = _row_probs(q[b, h, i], kh, i, causal, wl, scale)
                pmax = max(p.values())
                for c in range(d):
                    pv[b, h, i, c] = math.fsum(p[j] * abs(vh[j, c]) for j in vis)
                    tail[b, h, i, c] = math.fsum(min(p[j], frac * pmax) * abs(vh[j, c]) for j in vis)
                sabs[b, h, i] = max(abs(scale) * math.fsum(abs(q[b, h, i, c]) * abs(kh[j, c]) for c in range(d))
                                    for j in vis)
    return {"pv": pv, "tail": tail, "sabs": sabs}


def _head_terms(qh, kh, vh, doh, causal, wl, scale, shift=0):
    """Per query row of one head: (vis, p, dS, F) by loops; the row at index
    i stands at key position i + shift."""
    N, d = qh.shape
    rows = []
    for i in range(N):
        vis, p, _ = _row_probs(qh[i], kh, i + shift, causal, wl, scale)
        dP = {j: math.fsum(doh[i, c] * vh[j, c] for c in range(d)) for j in vis}
        D = math.fsum(p[j] * dP[j] for j in vis)
        dS = {j: p[j] * (dP[j] - D) for j in vis}
        F = math.fsum(abs(doh[i, c]) * math.fsum(p[j] * abs(vh[j, c]) for j in vis) for c in range(d))
        rows.append((vis, p, dS, F))
    return rows


def _group_mags(qs, kh, vh, dos, causal, wl, scale, shift=0):
    """Magnitudes of one key/value head and the G query heads of its group:
    dq, dq_f [G, N, d]; dk, dk_f, dv [Nk, d]."""
    G, N, d = qs.shape
    Nk = kh.shape[0]
    terms = [_head_terms(qs[gi], kh, vh, dos[gi], causal, wl, scale, shift) for gi in range(G)]
    dq = np.zeros((G, N, d))
    dq_f = np.zeros((G, N, d))
    for gi in range(G):
        for i, (vis, p, dS, F) in enumerate(terms[gi]):
            for c in range(d):
                dq[gi, i, c] = abs(scale) * math.fsum(abs(dS[j]) * abs(kh[j, c]) for j in vis)
                dq_f[gi, i, c] = abs(scale) * math.fsum(p[j] * F * abs(kh[j, c]) for j in vis)
    dq_v = np.zeros((G, N, d))
    for gi in range(G):
        for i, (vis, p, dS, F) in enumerate(terms[gi]):
            for c in range(d):
                dq_v[gi, i, c] = abs(scale) * math.fsum(abs(kh[j, c]) for j in vis)
    dk = np.zeros((Nk, d))
    dk_f = np.zeros((Nk, d))
    dv = np.zeros((Nk, d))
    dk_v = np.zeros((Nk, d))
    dv_v = np.zeros((Nk, d))
    for j in range(Nk):
        for c in range(d):
            a, bf, cv, kv, vv = [], [], [], [], []
            for gi in range(G):
                for i, (vis, p, dS, F) in enumerate(terms[gi]):
                    if j in p:
                        a.append(abs(dS[j]) * abs(qs[gi, i, c]))
                        bf.append(p[j] * F * abs(qs[gi, i, c]))
                        cv.append(p[j] * abs(dos[gi, i, c]))
                        kv.append(abs(qs[gi, i, c]))
                        vv.append(abs(dos[gi, i, c]))
            dk[j, c] = abs(scale) * math.fsum(a)
            dk_f[j, c] = abs(scale) * math.fsum(bf)
            dv[j, c] = math.fsum(cv)
            dk_v[j, c] = abs(scale) * math.fsum(kv)
            dv_v[j, c] = math.fsum(vv)
    return {"dq": dq, "dq_f": dq_f, "dk": dk, "dk_f": dk_f, "dv": dv, "dq_v": dq_v, "dk_v": dk_v, "dv_v": dv_v}


def bwd_mags_brute(q, k, v, do, causal, wl, scale):
    """The gradient oracle's magnitude terms, element by element."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = {"dq": np.zeros_like(q), "dq_f": np.zeros_like(q), "dk": np.zeros_like(k), "dk_f": np.zeros_like(k),
           "dv": np.zeros_like(v), "dq_v": np.zeros_like(q), "dk_v": np.zeros_like(k), "dv_v": np.zeros_like(v)}
    for b in range(B):
        for hk in range(Hkv):
            hs = slice(hk * G, (hk + 1) * G)
            m = _group_mags(q[b, hs], k[b, hk], v[b, hk], do[b, hs], causal, wl, scale)
            for key in ("dq", "dq_f", "dq_v"):
                out[key][b, hs] = m[key]
            for key in ("dk", "dk_f", "dv", "dk_v", "dv_v"):
                out[key][b, hk] = m[key]
    return out


def _close(got, want, what, rel=1e-12):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    tol = rel * max(1.0, float(np.abs(want).max(initial=0.0)))
    err = float(np.abs(got - want).max(initial=0.0))
    assert err <= tol, f"{what}: max error {err:.3e} > {tol:.3e}"


# ---------------------------------------------------------------------------
# Forward magnitudes: fwd_mag(q, k, v, causal, wl, scale, frac) -> (o, lse, mags)

def pin_fwd_mag_brute_force(fwd_mag):
    """Every forward magnitude equals its element-by-element brute force."""
    cases = [(1, 2, 1, 7, 3, 0.6, 2.0 ** -3), (2, 4, 2, 9, 4, 0.35, 0.5), (1, 3, 3, 5, 2, 1.3, 2.0 ** -10),
             (1, 2, 1, 6, 3, -0.7, 2.0 ** -2), (1, 2, 2, 5, 2, 0.0, 0.5)]
    for ci, (B, Hq, Hkv, N, d, scale, frac) in enumerate(cases):
        q, k, v = random_inputs(900 + ci, "f32", B, Hq, Hkv, N, d, mult=2.0)
        for causal, wl in MASKS:
            _, _, m = fwd_mag(q, k, v, causal, wl, scale, frac)
            want = fwd_mags_brute(q, k, v, causal, wl, scale, frac)
            for key in ("pv", "tail", "sabs"):
                _close(m[key], want[key], f"{key} case {ci} causal={causal} wl={wl}")


def pin_fwd_mag_closed_forms(fwd_mag):
    """V >= 0: P|V| = O.  Fraction >= 1: tail = P|V|.  Equal keys (uniform
    visible probabilities): tail = f P|V| for f < 1, and P|V| is the mean of
    the visible |V| rows."""
    B, Hq, Hkv, N, d = 1, 4, 2, 13, 5
    q, k, v = random_inputs(910, "f32", B, Hq, Hkv, N, d, mult=1.5)
    va = np.abs(v).astype(np.float64)
    for causal, wl in MASKS:
        o, _, m = fwd_mag(q, k, va, causal, wl, 0.8, 2.0 ** -6)
        _close(m["pv"], o, f"P|V| = O for V >= 0, causal={causal} wl={wl}")
        _, _, m1 = fwd_mag(q, k, v, causal, wl, 0.8, 1.0)
        _close(m1["tail"], m1["pv"], f"tail(1) = P|V|, causal={causal} wl={wl}")
        _, _, m2 = fwd_mag(q, k, v, causal, wl, 0.8, 3.0)
        _close(m2["tail"], m2["pv"], f"tail(3) = P|V|, causal={causal} wl={wl}")
    keq = np.repeat(k[:, :, :1], N, axis=2)
    for causal, wl in MASKS:
        for f in (0.25, 2.0 ** -9):
            _, _, m = fwd_mag(q, keq, v, causal, wl, 0.8, f)
            _close(m["tail"], f * m["pv"], f"tail = f P|V| for equal keys, causal={causal} wl={wl}")
            for i in range(N):
                vis = [j for j in range(N) if not _hidden(i, j, causal, wl)]
                for h in range(Hq):
                    _close(m["pv"][0, h, i], va[0, h // 2, vis].mean(axis=0), f"mean |V| row {i}")


# ---------------------------------------------------------------------------
# Gradient magnitudes: bwd_mag(q, k, v, do, causal, wl, scale) -> (dq, dk, dv, mags)

def pin_bwd_mag_brute_force(bwd_mag):
    """Every gradient magnitude equals its element-by-element brute force
    (GQA groups of 1 and 2, every mask kind)."""
    cases = [(1, 2, 1, 6, 3, 0.7), (1, 2, 2, 5, 4, 1.1), (2, 4, 2, 4, 2, 0.45), (1, 2, 1, 5, 3, -0.9),
             (1, 4, 2, 4, 2, -0.3)]
    for ci, (B, Hq, Hkv, N, d, scale) in enumerate(cases):
        q, k, v = random_inputs(920 + ci, "f32", B, Hq, Hkv, N, d, mult=1.5)
        do = np.random.default_rng(930 + ci).standard_normal((B, Hq, N, d))
        for causal, wl in MASKS:
            m = bwd_mag(q, k, v, do, causal, wl, scale)[3]
            want = bwd_mags_brute(q, k, v, do, causal, wl, scale)
            for key in ("dq", "dk", "dv", "dq_f", "dk_f", "dq_v", "dk_v", "dv_v"):
                _close(m[key], want[key], f"{key} case {ci} causal={causal} wl={wl}")


def pin_bwd_mag_closed_forms(bwd_mag):
    """dO >= 0: P^T|dO| = dV.  dO, V >= 0 and K all ones: the dq_f row is
    scale * sum_c do_ic o_ic in every column.  Q all ones with equal keys:
    dk_f_j = scale * sum over the rows i that see j of F_i / n_i."""
    from oracle import attention_fwd

    B, Hq, Hkv, N, d = 1, 4, 2, 11, 3
    q, k, v = random_inputs(940, "f32", B, Hq, Hkv, N, d)
    do = np.random.default_rng(941).standard_normal((B, Hq, N, d))
    da, va = np.abs(do), np.abs(v).astype(np.float64)
    ones_k = np.ones_like(k, dtype=np.float64)
    G = Hq // Hkv
    for causal, wl in MASKS:
        _, _, dv, m = bwd_mag(q, k, v, da, causal, wl, 0.6)
        _close(m["dv"], dv, f"P^T|dO| = dV for dO >= 0, causal={causal} wl={wl}")
        _, _, _, m = bwd_mag(q, ones_k, va, da, causal, wl, 0.6)
        o, _ = attention_fwd(q, ones_k, va, causal, wl, 0.6, threads=1)
        rowterm = (da * o).sum(axis=-1)
        _close(m["dq_f"], 0.6 * np.repeat(rowterm[..., None], d, axis=-1),
               f"dq_f with K = 1, causal={causal} wl={wl}")
        # equal keys: p_ij = 1/n_i on the visible keys, whatever q is
        q1 = np.ones_like(q, dtype=np.float64)
        keq = np.repeat(k[:, :, :1], N, axis=2)
        _, _, _, m = bwd_mag(q1, keq, va, da, causal, wl, 0.6)
        o, _ = attention_fwd(q1, keq, va, causal, wl, 0.6, threads=1)
        F = (da * o).sum(axis=-1)                   # V >= 0: P|V| = O
        for hk in range(Hkv):
            for j in range(N):
                rows = [(h, i) for h in range(hk * G, (hk + 1) * G) for i in range(N)
                        if not _hidden(i, j, causal, wl)]
                n = {i: sum(1 for jj in range(N) if not _hidden(i, jj, causal, wl)) for _, i in rows}
                want = 0.6 * math.fsum(F[0, h, i] / n[i] for h, i in rows)
                _close(m["dk_f"][0, hk, j], np.full(d, want), f"dk_f equal keys j={j} causal={causal} wl={wl}")


def pin_bwd_mag_visibility(bwd_mag):
    """The visibility products: with no mask every key is visible to every
    query, so dv_v_j = sum over the group's rows of |dO| and dq_v_i =
    |scale| sum_j |K_j| for every row; a causal mask gives key j the rows
    i >= j and row i the keys j <= i (prefix and suffix sums); the window of
    0 keys (with causal) leaves only the diagonal."""
    B, Hq, Hkv, N, d = 1, 4, 2, 9, 3
    q, k, v = random_inputs(960, "f32", B, Hq, Hkv, N, d)
    do = np.random.default_rng(961).standard_normal((B, Hq, N, d))
    G = Hq // Hkv
    aq, ak, ado = np.abs(q).astype(np.float64), np.abs(k).astype(np.float64), np.abs(do)
    for scale in (0.7, -0.4):
        m = bwd_mag(q, k, v, do, False, -1, scale)[3]
        for hk in range(Hkv):
            grp = slice(hk * G, (hk + 1) * G)
            _close(m["dv_v"][0, hk], np.broadcast_to(ado[0, grp].sum(axis=(0, 1)), (N, d)), "dv_v no mask")
            _close(m["dk_v"][0, hk], np.broadcast_to(abs(scale) * aq[0, grp].sum(axis=(0, 1)), (N, d)), "dk_v no mask")
            for h in range(hk * G, (hk + 1) * G):
                _close(m["dq_v"][0, h], np.broadcast_to(abs(scale) * ak[0, hk].sum(axis=0), (N, d)), "dq_v no mask")
        m = bwd_mag(q, k, v, do, True, -1, scale)[3]
        for hk in range(Hkv):
            grp = slice(hk * G, (hk + 1) * G)
            suffix = np.cumsum(ado[0, grp].sum(axis=0)[::-1], axis=0)[::-1]
            _close(m["dv_v"][0, hk], suffix, "dv_v causal")
            for h in range(hk * G, (hk + 1) * G):
                _close(m["dq_v"][0, h], abs(scale) * np.cumsum(ak[0, hk], axis=0), "dq_v causal")
        m = bwd_mag(q, k, v, do, True, 0, scale)[3]
        for hk in range(Hkv):
            _close(m["dv_v"][0, hk], ado[0, hk * G:(hk + 1) * G].sum(axis=0), "dv_v diagonal")
            _close(m["dk_v"][0, hk], abs(scale) * aq[0, hk * G:(hk + 1) * G].sum(axis=0), "dk_v diagonal")


def pin_bwd_mag_two_keys(bwd_mag):
    """Causal row 1 sees keys 0 and 1 only: with a = s_10 - s_11,
    p_10 = 1 / (1 + e^-a), p_11 = 1 - p_10, and |dS_10| = |dS_11| =
    p_10 p_11 |<do_1, v_0 - v_1>|.  Row 0 sees one key, so its dS is 0.
    With K all ones (the scores tie, p = 1/2) dq row 1 is scale * 2 |dS_10| in
    every column; with Q all ones dk row j is scale |dS_1j| in every column."""
    d = 4
    rng = np.random.default_rng(950)
    v = rng.standard_normal((1, 1, 2, d))
    do = rng.standard_normal((1, 1, 2, d))
    scale = 0.9
    # K = 1: scores tie, p = 1/2 each
    q = rng.standard_normal((1, 1, 2, d))
    k1 = np.ones((1, 1, 2, d))
    m = bwd_mag(q, k1, v, do, True, -1, scale)[3]
    ds = 0.25 * abs(float(do[0, 0, 1] @ (v[0, 0, 0] - v[0, 0, 1])))
    _close(m["dq"][0, 0, 1], np.full(d, scale * 2 * ds), "dq row 1 with K = 1")
    _close(m["dq"][0, 0, 0], np.zeros(d), "dq row 0 (one visible key)")
    # Q = 1: p_10 is the logistic function of scale * (sum k_0 - sum k_1)
    q1 = np.ones((1, 1, 2, d))
    k = rng.standard_normal((1, 1, 2, d))
    a = scale * (float(k[0, 0, 0].sum()) - float(k[0, 0, 1].sum()))
    p0 = 1.0 / (1.0 + math.exp(-a))
    ds = p0 * (1.0 - p0) * abs(float(do[0, 0, 1] @ (v[0, 0, 0] - v[0, 0, 1])))
    m = bwd_mag(q1, k, v, do, True, -1, scale)[3]
    for j in range(2):
        _close(m["dk"][0, 0, j], np.full(d, scale * ds), f"dk row {j} with Q = 1")


# ---------------------------------------------------------------------------
# Packed sequences: bwd_varlen_mag(q, k, v, do, cu_q, cu_k, causal=, window_left=,
# scale=) -> (dq, dk, dv, mags), laid out [total][H][d]

def pin_varlen_bwd_mag_brute_force(bwd_varlen_mag):
    """The packed gradient oracle's magnitudes equal the brute force of each
    sequence, its queries at the end of its keys (fewer, as many and more
    queries than keys; a row that sees no key has zero magnitudes)."""
    lens = [(2, 4), (3, 3), (3, 1), (0, 2)]
    cq = np.cumsum([0] + [a for a, _ in lens])
    ck = np.cumsum([0] + [b for _, b in lens])
    Hq, Hkv, d = 2, 1, 3
    rng = np.random.default_rng(960)
    q = rng.standard_normal((cq[-1], Hq, d))
    k = rng.standard_normal((ck[-1], Hkv, d))
    v = rng.standard_normal((ck[-1], Hkv, d))
    do = rng.standard_normal((cq[-1], Hq, d))
    for causal, wl in [(False, -1), (True, -1), (True, 1), (False, 0)]:
        m = bwd_varlen_mag(q, k, v, do, cq, ck, causal=causal, window_left=wl, scale=0.8)[3]
        for b, (lq, lk) in enumerate(lens):
            a, z, ka, kz = cq[b], cq[b + 1], ck[b], ck[b + 1]
            for hk in range(Hkv):
                hs = slice(hk * (Hq // Hkv), (hk + 1) * (Hq // Hkv))
                want = _group_mags(q[a:z, hs].transpose(1, 0, 2), k[ka:kz, hk], v[ka:kz, hk],
                                   do[a:z, hs].transpose(1, 0, 2), causal, wl, 0.8, shift=lk - lq)
                for key in ("dq", "dq_f", "dq_v"):
                    _close(m[key][a:z, hs].transpose(1, 0, 2), want[key], f"{key} sequence {b} c={causal} wl={wl}")
                for key in ("dk", "dk_f", "dv", "dk_v", "dv_v"):
                    _close(m[key][ka:kz, hk], want[key], f"{key} sequence {b} c={causal} wl={wl}")


FWD_MAG_PINS = [pin_fwd_mag_brute_force, pin_fwd_mag_closed_forms]
BWD_MAG_PINS = [pin_bwd_mag_brute_force, pin_bwd_mag_closed_forms, pin_bwd_mag_visibility, pin_bwd_mag_two_keys]
VARLEN_BWD_MAG_PINS = [pin_varlen_bwd_mag_brute_force]
