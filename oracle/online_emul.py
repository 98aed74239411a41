"""The tiled, online-softmax form of exact attention in fp64 (test
infrastructure only; see package doc).

Steps, in the order the pages give them:
  * Q, K and V are split into blocks (Flash Attention page, heepie.pages.dev,
    tiling section): Br query rows per query block, Bc keys per key/value
    block.
  * Per query block, a partial result and its normalisation factors stay
    "on chip" while key/value blocks stream past ("TO-BE" diagram): a running
    row max m, a running row sum l of exp(s - m), and the unnormalised
    partial output acc.
  * Each new block's scores are folded in with the online (incremental)
    softmax of the FlashAttention quiz, question 4: when the row max grows
    from m to m', everything accumulated so far is rescaled by exp(m - m').
  * After the last block the partial output is divided by l once; the row
    logsumexp is m + log l.

In real arithmetic this equals the standard definition exactly (the pages'
"exact, not approximate" claim): exp(x - m') = exp(x - m) * exp(m - m').
The block order within a query block is ascending, and blocks in which every
(query, key) pair is masked may be skipped -- they would contribute rescale
factor 1 and zero probabilities.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention_ref import kv_head_of, masked


def attention_online(q, k, v, causal: bool = False, window_left: int = -1,
                     scale: Optional[float] = None, Br: int = 64, Bc: int = 64,
                     skip_masked_blocks: bool = True):
    """Returns (o [B,Hq,N,d] fp64, lse [B,Hq,N] fp64) computed block-wise."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, N, Br):
                rows = np.arange(r0, min(r0 + Br, N))
                Qb = q[b, h, rows]
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), d))
                for c0 in range(0, N, Bc):
                    cols = np.arange(c0, min(c0 + Bc, N))
                    hide = masked(rows[:, None], cols[None, :], causal, window_left)
                    if skip_masked_blocks and hide.all():
                        continue
                    S = scale * (Qb @ k[b, hk, cols].T)
                    S[hide] = -np.inf
                    m_new = np.maximum(m, S.max(axis=1))
                    # rows with nothing visible yet keep m = -inf: use 0 as the
                    # shift so that exp gives 0 rather than nan
                    shift = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.exp(m - shift)
                    P = np.exp(S - shift[:, None])
                    l = alpha * l + P.sum(axis=1)
                    acc = alpha[:, None] * acc + P @ v[b, hk, cols]
                    m = m_new
                o[b, h, rows] = acc / l[:, None]
                lse[b, h, rows] = m + np.log(l)
    return o, lse
