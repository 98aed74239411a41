"""Exact attention as explicit Python loops (test infrastructure only).

A second, independent spelling of the definition in the package doc, for tiny
inputs: for each query row, pass 1 finds the largest visible scaled score;
pass 2 sums exp(score - max) over the visible keys and accumulates the
exp-weighted value rows; the output is that weighted sum over the exp sum.
No numpy linear algebra: dot products are written out with math.fsum, so a
transposed operand or a wrong head index in the vectorised oracle cannot be
mirrored here.
"""
from __future__ import annotations

import math
from typing import Optional


def attention_twopass(q, k, v, causal: bool = False, window_left: int = -1,
                      scale: Optional[float] = None):
    """q: nested lists / array [B][Hq][N][d]; k, v: [B][Hkv][N][d].

    Returns (o, lse) as nested Python lists of floats, o [B][Hq][N][d],
    lse [B][Hq][N].
    """
    B = len(q)
    Hq = len(q[0]) if B else 0
    Hkv = len(k[0]) if B else 0
    N = len(q[0][0]) if B and Hq else 0
    d = len(q[0][0][0]) if N else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = Hq // Hkv if Hkv else 1
    o = [[[[0.0] * d for _ in range(N)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for i in range(N):
                vis = []
                for j in range(N):
                    if causal and j > i:
                        continue
                    if window_left >= 0 and j < i - window_left:
                        continue
                    vis.append(j)
                scores = {}
                for j in vis:
                    scores[j] = scale * math.fsum(float(q[b][h][i][c]) * float(k[b][hk][j][c])
                                                  for c in range(d))
                # pass 1: the row max
                mx = max(scores.values())
                # pass 2: exp-sum and exp-weighted value sum
                w = {j: math.exp(scores[j] - mx) for j in vis}
                z = math.fsum(w.values())
                for c in range(d):
                    o[b][h][i][c] = math.fsum(w[j] * float(v[b][hk][j][c]) for j in vis) / z
                lse[b][h][i] = mx + math.log(z)
    return o, lse
