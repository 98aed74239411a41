"""Plain fp64 gradients of exact attention (test infrastructure only).

What is differentiated is the forward of ``attention_ref``: for batch b, query
head h (key/value head h_kv = h // (Hq // Hkv)) and query row i,

    s_ij = scale * <q_i, k_j>,   s_ij = -inf where masked,
    p_ij = softmax_j(s_ij),      o_i = sum_j p_ij v_j.

Given an upstream gradient dO of the output (the logsumexp output carries no
upstream gradient), the chain rule gives, per (b, h),

    dV   = P^T dO                       (o is linear in v)
    dP   = dO V^T                       (dL/dp_ij = <do_i, v_j>)
    dS   = P * (dP - rowsum(P * dP))    (Jacobian of a row softmax)
    dQ   = scale * dS K
    dK   = scale * dS^T Q

and a key/value head shared by a group of query heads collects the dK and dV
of every head in its group (the same K/V rows enter each of those heads'
forward).  Masked pairs have p_ij = 0, so they contribute nothing anywhere.

This is the backward pass the Flash Attention page alludes to in its tiling
section ("recomputation": the probabilities are rebuilt from Q, K and the
saved row statistics instead of being stored); the oracle simply materialises
P per block of query rows, over every key, in fp64.  The pages print no
backward formulas: the ones above are the derivative of the forward, which is
the plainest reading of "the gradient of exact attention".

Optionally the function also returns, for error bounds in tests, the same
products taken over absolute values (|P|^T |dO|, |scale| |dS| |K|,
|scale| |dS|^T |Q|) and the row terms F_i = sum_c |do_ic| (P |V|)_ic -- a
bound on sum_c |do_ic| |o_ic| that also covers a rounded P inside o -- with
their products |scale| (P * F) |K| and |scale| (P * F)^T |Q|; and the same
products with P and dS replaced by the visibility matrix (1 where key j is
visible to query i, else 0): Vis^T |dO|, |scale| Vis |K|, |scale| Vis^T |Q|
('dv_v', 'dq_v', 'dk_v'), the sums an absolute per-entry error of P or dS
can reach.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from .attention_ref import kv_head_of, masked

ROW_BLOCK = 256


def _one_kv_head(qs, kh, vh, dos, causal, window_left, scale, bounds, shift=0):
    """Gradients for one (batch, key/value head) and the query heads of its
    group.  qs, dos: [G, N, d] fp64; kh, vh: [Nk, d] fp64 (Nk = N for
    self-attention).  Query row i stands at key position i + shift (0 for
    self-attention; Nk - N when the queries are the last tokens of a longer
    sequence); a row that sees no key has P = 0 and passes no gradient.
    Returns dq [G, N, d], dk [Nk, d], dv [Nk, d] and, if bounds, a dict of
    magnitude terms."""
    G, N, d = qs.shape
    Nk = kh.shape[0]
    keys = np.arange(Nk)
    dq = np.zeros((G, N, d))
    dk = np.zeros((Nk, d))
    dv = np.zeros((Nk, d))
    mag = None
    if bounds:
        mag = {"dq": np.zeros((G, N, d)), "dk": np.zeros((Nk, d)), "dv": np.zeros((Nk, d)),
               "dq_f": np.zeros((G, N, d)), "dk_f": np.zeros((Nk, d)),
               "dq_v": np.zeros((G, N, d)), "dk_v": np.zeros((Nk, d)), "dv_v": np.zeros((Nk, d))}
    if Nk == 0:
        return dq, dk, dv, mag
    for g in range(G):
        qh, doh = qs[g], dos[g]
        for s0 in range(0, N, ROW_BLOCK):
            r = np.arange(s0, min(N, s0 + ROW_BLOCK))
            pos = r + shift
            # recompute the probabilities of these rows against every key
            S = scale * (qh[r] @ kh.T)
            hidden = masked(pos[:, None], keys[None, :], causal, window_left)
            S[hidden] = -np.inf
            m = S.max(axis=1, keepdims=True)
            m[~np.isfinite(m)] = 0.0  # a row that sees no key: every E below is 0
            E = np.exp(S - m)
            z = E.sum(axis=1, keepdims=True)
            P = E / np.where(z > 0, z, 1.0)
            # chain rule through O = P V and the row softmax
            dv += P.T @ doh[r]
            dP = doh[r] @ vh.T
            rowdot = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - rowdot)
            dq[g, r] = scale * (dS @ kh)
            dk += scale * (dS.T @ qh[r])
            if bounds:
                A = np.abs(dS)
                mag["dv"] += P.T @ np.abs(doh[r])
                mag["dq"][g, r] = abs(scale) * (A @ np.abs(kh))
                mag["dk"] += abs(scale) * (A.T @ np.abs(qh[r]))
                F = (np.abs(doh[r]) * (P @ np.abs(vh))).sum(axis=1, keepdims=True)
                PF = P * F
                mag["dq_f"][g, r] = abs(scale) * (PF @ np.abs(kh))
                mag["dk_f"] += abs(scale) * (PF.T @ np.abs(qh[r]))
                Vis = (~hidden).astype(np.float64)
                mag["dv_v"] += Vis.T @ np.abs(doh[r])
                mag["dq_v"][g, r] = abs(scale) * (Vis @ np.abs(kh))
                mag["dk_v"] += abs(scale) * (Vis.T @ np.abs(qh[r]))
    return dq, dk, dv, mag


def attention_bwd(q, k, v, do, causal: bool = False, window_left: int = -1,
                  scale: Optional[float] = None, threads: Optional[int] = None,
                  bounds: bool = False):
    """Exact attention gradients in float64.

    q, do: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float dtype; widened to
    fp64).  Returns (dq [B, Hq, N, d], dk [B, Hkv, N, d], dv [B, Hkv, N, d]),
    plus a dict of magnitude terms (same keys as the gradients, and 'dq_f',
    'dk_f'; shapes as the gradient they bound) when bounds=True.

    Raises ValueError on inconsistent shapes, Hq not a multiple of Hkv, or
    window_left < -1.
    """
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or do.shape != q.shape:
        raise ValueError("q, do must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if (Bk, Nk, dk_) != (B, N, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    if window_left < -1:
        raise ValueError("window_left must be >= -1")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scale = float(scale)
    G = Hq // Hkv
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    mags = None
    if bounds:
        mags = {"dq": np.zeros_like(dq), "dk": np.zeros_like(dk), "dv": np.zeros_like(dv),
                "dq_f": np.zeros_like(dq), "dk_f": np.zeros_like(dk),
                "dq_v": np.zeros_like(dq), "dk_v": np.zeros_like(dk), "dv_v": np.zeros_like(dv)}
    if B * Hq * N == 0:
        return (dq, dk, dv, mags) if bounds else (dq, dk, dv)

    def work(bk):
        b, hk = divmod(bk, Hkv)
        heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == hk]
        qs = np.stack([q[b, h].astype(np.float64) for h in heads])
        dos = np.stack([do[b, h].astype(np.float64) for h in heads])
        gq, gk, gv, mag = _one_kv_head(qs, k[b, hk].astype(np.float64), v[b, hk].astype(np.float64), dos,
                                       causal, window_left, scale, bounds)
        for gi, h in enumerate(heads):
            dq[b, h] = gq[gi]
            if bounds:
                for key in ("dq", "dq_f", "dq_v"):
                    mags[key][b, h] = mag[key][gi]
        dk[b, hk] = gk
        dv[b, hk] = gv
        if bounds:
            for key in ("dk", "dv", "dk_f", "dk_v", "dv_v"):
                mags[key][b, hk] = mag[key]

    nthreads = threads or len(os.sched_getaffinity(0))
    nthreads = max(1, min(nthreads, B * Hkv))
    if nthreads == 1:
        for bk in range(B * Hkv):
            work(bk)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(B * Hkv)))
    return (dq, dk, dv, mags) if bounds else (dq, dk, dv)


def attention_bwd_varlen(q, k, v, do, cu_seqlens_q, cu_seqlens_k, causal: bool = False, window_left: int = -1,
                         scale: Optional[float] = None, threads: Optional[int] = None, bounds: bool = False):
    """Gradients of ``attention_fwd_varlen`` (packed sequences) in float64.

    q, do: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; sequence b owns query
    rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b]
    .. cu_seqlens_k[b+1]-1, its Lq query rows standing at the end of its Lk
    keys (row i at key position Lk - Lq + i).  Within each sequence this is
    ``attention_bwd`` with that alignment; rows that see no key pass no
    gradient.  Returns (dq [total_q, Hq, d], dk [total_k, Hkv, d],
    dv [total_k, Hkv, d]), plus the magnitude terms (laid out like the
    gradients) when bounds=True.
    """
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or q.shape[2] != k.shape[2] or do.shape != q.shape:
        raise ValueError("q, do must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    if len(cq) != len(ck) or len(cq) < 1 or cq[0] != 0 or ck[0] != 0 or cq[-1] != q.shape[0] \
            or ck[-1] != k.shape[0] or any(b < a for a, b in zip(cq, cq[1:])) or any(b < a for a, b in zip(ck, ck[1:])):
        raise ValueError("cu_seqlens must be nondecreasing prefix sums from 0 to the packed lengths")
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    if window_left < -1:
        raise ValueError("window_left must be >= -1")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scale = float(scale)
    dq = np.zeros((q.shape[0], Hq, d))
    dk = np.zeros((k.shape[0], Hkv, d))
    dv = np.zeros((k.shape[0], Hkv, d))
    mags = None
    if bounds:
        mags = {"dq": np.zeros_like(dq), "dk": np.zeros_like(dk), "dv": np.zeros_like(dv),
                "dq_f": np.zeros_like(dq), "dk_f": np.zeros_like(dk),
                "dq_v": np.zeros_like(dq), "dk_v": np.zeros_like(dk), "dv_v": np.zeros_like(dv)}

    def work(bk):
        b, hk = divmod(bk, Hkv)
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == hk]
        qs = np.stack([q[q0:q1, h].astype(np.float64) for h in heads])
        dos = np.stack([do[q0:q1, h].astype(np.float64) for h in heads])
        gq, gk, gv, mag = _one_kv_head(qs, k[k0:k1, hk].astype(np.float64), v[k0:k1, hk].astype(np.float64), dos,
                                       causal, window_left, scale, bounds, shift=(k1 - k0) - (q1 - q0))
        for gi, h in enumerate(heads):
            dq[q0:q1, h] = gq[gi]
            if bounds:
                mags["dq"][q0:q1, h] = mag["dq"][gi]
                mags["dq_f"][q0:q1, h] = mag["dq_f"][gi]
                mags["dq_v"][q0:q1, h] = mag["dq_v"][gi]
        dk[k0:k1, hk] = gk
        dv[k0:k1, hk] = gv
        if bounds:
            mags["dk"][k0:k1, hk] = mag["dk"]
            mags["dv"][k0:k1, hk] = mag["dv"]
            mags["dk_f"][k0:k1, hk] = mag["dk_f"]
            mags["dk_v"][k0:k1, hk] = mag["dk_v"]
            mags["dv_v"][k0:k1, hk] = mag["dv_v"]

    n = (len(cq) - 1) * Hkv
    nthreads = max(1, min(threads or len(os.sched_getaffinity(0)), max(n, 1)))
    if nthreads == 1:
        for bk in range(n):
            work(bk)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(n)))
    return (dq, dk, dv, mags) if bounds else (dq, dk, dv)
