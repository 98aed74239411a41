"""Plain fp64 attention of a few new query rows against a key/value cache
(test infrastructure only; see package doc).

The setting is inference: a sequence of L_b tokens has its keys and values in
a cache, and its last Nq tokens ask queries.  Query row i of batch b stands at
position p = L_b - Nq + i of that sequence (the rows are aligned to the end
of the cache, "bottom-right"), so under a causal mask it sees the cached keys
j <= p, exactly as row p of causal self-attention over the whole sequence
would.  For batch b, query head h (key/value head h // (Hq // Hkv)):

    s_ij = scale * <q[b,h,i,:], k[b,h_kv,j,:]>      for j < L_b
    (i, j) masked when j >= L_b, (causal and j > p), or
                       (window_left >= 0 and j < p - window_left)
    o[b,h,i,:] = sum_j softmax_j(s_i.) v[b,h_kv,j,:],  lse = log sum_j exp(s_ij)

A row that sees no key (p < 0 under a causal mask, or L_b = 0) has o = 0 and
lse = -inf, the values an empty sum gives.

Sources: the same definition as ``attention_ref`` (Flash Attention page,
"AS-IS" diagram; Hacker News answers on GQA and on windows as masks).  The
pages name inference and decoding only in passing (the Hacker News thread on
llama.cpp, the FastAttention abstract's inference focus, the FlashDecoding++
title in the FA2 article's literature list); the end alignment, the per-batch
cache lengths and the empty-row convention are readings of this library.
S and P are materialised per (batch, head) over every cached key.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

from .attention_ref import kv_head_of


def visible_keys(L: int, Nq: int, causal: bool, window_left: int) -> np.ndarray:
    """[Nq, L] boolean: True where query row i (at position L - Nq + i) may
    see cached key j (< L)."""
    p = (L - Nq + np.arange(Nq))[:, None]
    j = np.arange(L)[None, :]
    vis = np.ones((Nq, L), dtype=bool)
    if causal:
        vis &= j <= p
    if window_left >= 0:
        vis &= j >= p - window_left
    return vis


def attention_fwd_kvcache(q, k, v, seqlens: Optional[Sequence[int]] = None, causal: bool = False,
                          window_left: int = -1, scale: Optional[float] = None, threads: Optional[int] = None):
    """Attention of q against the first seqlens[b] cached keys of batch b.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] (the cache, logically contiguous;
    any float dtype, widened to fp64); seqlens: B lengths in [0, Nk], or None
    for Nk everywhere.  Returns (o [B, Hq, Nq, d], lse [B, Hq, Nq]) in fp64,
    with o = 0 and lse = -inf on rows that see no key.

    Raises ValueError on inconsistent shapes, Hq not a multiple of Hkv,
    window_left < -1 or a length outside [0, Nk].
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("shape mismatch")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    if window_left < -1:
        raise ValueError("window_left must be >= -1")
    lens = [Nk] * B if seqlens is None else [int(x) for x in seqlens]
    if len(lens) != B or any(not 0 <= L <= Nk for L in lens):
        raise ValueError("seqlens must hold B lengths in [0, Nk]")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scale = float(scale)
    o = np.zeros((B, Hq, Nq, d), dtype=np.float64)
    lse = np.full((B, Hq, Nq), -np.inf, dtype=np.float64)

    def work(bh):
        b, h = divmod(bh, Hq)
        L = lens[b]
        if L == 0 or Nq == 0:
            return
        hk = kv_head_of(h, Hq, Hkv)
        kh = k[b, hk, :L].astype(np.float64)
        vh = v[b, hk, :L].astype(np.float64)
        S = scale * (q[b, h].astype(np.float64) @ kh.T)
        vis = visible_keys(L, Nq, causal, window_left)
        S[~vis] = -np.inf
        rows = vis.any(axis=1)          # rows that see at least one key
        if not rows.any():
            return
        Sr = S[rows]
        m = Sr.max(axis=1, keepdims=True)
        E = np.exp(Sr - m)
        z = E.sum(axis=1, keepdims=True)
        o[b, h, rows] = (E / z) @ vh
        lse[b, h, rows] = m[:, 0] + np.log(z[:, 0])

    n = B * Hq
    nthreads = max(1, min(threads or len(os.sched_getaffinity(0)), n))
    if nthreads == 1:
        for bh in range(n):
            work(bh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(n)))
    return o, lse


def attention_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool = False, window_left: int = -1,
                         scale: Optional[float] = None, threads: Optional[int] = None):
    """Attention over a batch of sequences of different lengths, packed.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; sequence b owns query rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
    cu_seqlens_k[b+1]-1.  Each sequence is the cache case above with its own
    Lq rows against its own Lk keys (rows aligned to the end of the keys; with
    Lq = Lk this is ordinary self-attention).  Returns (o [total_q, Hq, d],
    lse [Hq, total_q]); rows that see no key get o = 0, lse = -inf.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    if len(cq) != len(ck) or len(cq) < 1 or cq[0] != 0 or ck[0] != 0 or cq[-1] != q.shape[0] \
            or ck[-1] != k.shape[0] or any(b < a for a, b in zip(cq, cq[1:])) or any(b < a for a, b in zip(ck, ck[1:])):
        raise ValueError("cu_seqlens must be nondecreasing prefix sums from 0 to the packed lengths")
    Hq, d = q.shape[1], q.shape[2]
    o = np.zeros((q.shape[0], Hq, d), dtype=np.float64)
    lse = np.full((Hq, q.shape[0]), -np.inf, dtype=np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0:
            continue
        qb = q[q0:q1].transpose(1, 0, 2)[None]          # [1, Hq, Lq, d]
        kb = k[k0:k1].transpose(1, 0, 2)[None]          # [1, Hkv, Lk, d]
        vb = v[k0:k1].transpose(1, 0, 2)[None]
        ob, lb = attention_fwd_kvcache(qb, kb, vb, None, causal, window_left, scale, threads)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[:, q0:q1] = lb[0]
    return o, lse
