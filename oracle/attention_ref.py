"""Plain fp64 standard attention (test infrastructure only; see package doc).

Follows the three phases of the "AS-IS" standard-attention diagram on the
Flash Attention page (heepie.pages.dev): scores S = Q K^T, probabilities
P = softmax(S) row-wise, output O = P V -- here with the scale applied to the
scores and the mask applied before the softmax, as the Hacker News answer on
sliding windows describes a window (the mask decides which queries see which
keys).  S and P are materialised for a block of query rows against every key.

Numbers: float64 throughout; inputs are widened from their storage type
(exact for f32/f16/bf16).  numpy's BLAS supplies the two matrix products.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

ROW_BLOCK = 256


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head used by query head ``h``: consecutive groups of
    Hq/Hkv query heads share one key/value head (grouped-query attention,
    Hacker News answer on GQA)."""
    return h // (Hq // Hkv)


def masked(i: np.ndarray, j: np.ndarray, causal: bool, window_left: int) -> np.ndarray:
    """True where query i may NOT see key j.

    causal: keys after the query are hidden (j > i).
    window_left >= 0: keys more than window_left positions before the query
    are hidden (j < i - window_left), so each query sees window_left + 1 keys
    ending at itself (fewer near the start).  -1 disables the window.
    """
    m = np.zeros(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        m |= j > i
    if window_left >= 0:
        m |= j < i - window_left
    return m


def _one_head(qh, kh, vh, rows, causal, window_left, scale, tail=None):
    """Attention for one (batch, query head): returns (O rows, lse rows) and,
    when ``tail`` is given, the magnitude rows (P|V|, sum_j min(p_ij,
    tail * max_j p_ij) |v_j|)."""
    N = kh.shape[0]
    d = vh.shape[1]
    out_o = np.empty((len(rows), d), dtype=np.float64)
    out_l = np.empty(len(rows), dtype=np.float64)
    mag_pv = np.empty((len(rows), d), dtype=np.float64) if tail is not None else None
    mag_tail = np.empty((len(rows), d), dtype=np.float64) if tail is not None else None
    mag_s = np.empty(len(rows), dtype=np.float64) if tail is not None else None
    keys = np.arange(N)
    for s0 in range(0, len(rows), ROW_BLOCK):
        r = rows[s0:s0 + ROW_BLOCK]
        # phase 1: S = scale * Q K^T for these rows against every key
        S = scale * (qh[r] @ kh.T)
        S[masked(r[:, None], keys[None, :], causal, window_left)] = -np.inf
        # phase 2: P = softmax(S), row-wise, shifted by the row max for range
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        z = E.sum(axis=1, keepdims=True)
        P = E / z
        # phase 3: O = P V
        out_o[s0:s0 + len(r)] = P @ vh
        out_l[s0:s0 + len(r)] = m[:, 0] + np.log(z[:, 0])
        if tail is not None:
            mag_pv[s0:s0 + len(r)] = P @ np.abs(vh)
            small = np.minimum(P, tail * P.max(axis=1, keepdims=True))
            mag_tail[s0:s0 + len(r)] = small @ np.abs(vh)
            A = abs(scale) * (np.abs(qh[r]) @ np.abs(kh).T)
            A[masked(r[:, None], keys[None, :], causal, window_left)] = 0.0
            mag_s[s0:s0 + len(r)] = A.max(axis=1)
    if tail is not None:
        return out_o, out_l, mag_pv, mag_tail, mag_s
    return out_o, out_l


def attention_fwd(q, k, v, causal: bool = False, window_left: int = -1,
                  scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None, tail: Optional[float] = None):
    """Exact attention forward in float64.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float dtype; widened to fp64).
    rows: optional query-row indices to evaluate (same for every head); the
    default is every row.  Returns (o [B, Hq, R, d] fp64, lse [B, Hq, R] fp64)
    where R = len(rows).

    With ``tail`` (a fraction), also returns a dict of magnitudes for error
    bounds, shaped like o: 'pv' = P|V| and 'tail' = sum_j min(p_ij, tail *
    max_j p_ij) |v_j| (the mass of probabilities below that fraction of their
    row's largest, as if dropped, bounded by it), shaped like o, and 'sabs' =
    max over visible j of |scale| * sum_c |q_ic| |k_jc|, shaped like lse (a
    bound on every visible score's size and on what its sum accumulates).

    Raises ValueError on inconsistent shapes, Hq not a multiple of Hkv, or
    window_left < -1.  Every row has at least one visible key (key j = i is
    never masked), so no empty-row convention is needed.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    if window_left < -1:
        raise ValueError("window_left must be >= -1")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scale = float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    o = np.empty((B, Hq, R, d), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    mags = {"pv": np.empty_like(o), "tail": np.empty_like(o), "sabs": np.empty_like(lse)} if tail is not None else None
    if B * Hq * R == 0:
        return (o, lse, mags) if tail is not None else (o, lse)

    def work(bh):
        b, h = divmod(bh, Hq)
        hk = kv_head_of(h, Hq, Hkv)
        qh = q[b, h].astype(np.float64)
        kh = k[b, hk].astype(np.float64)
        vh = v[b, hk].astype(np.float64)
        res = _one_head(qh, kh, vh, rows, causal, window_left, scale, tail)
        o[b, h], lse[b, h] = res[0], res[1]
        if tail is not None:
            mags["pv"][b, h], mags["tail"][b, h], mags["sabs"][b, h] = res[2], res[3], res[4]

    nthreads = threads or len(os.sched_getaffinity(0))
    nthreads = max(1, min(nthreads, B * Hq))
    if nthreads == 1:
        for bh in range(B * Hq):
            work(bh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(B * Hq)))
    return (o, lse, mags) if tail is not None else (o, lse)
