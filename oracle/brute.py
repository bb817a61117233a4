"""Scalar brute-force attention for tiny shapes (TEST INFRASTRUCTURE ONLY).

Written separately from ``oracle.ref`` and used to pin it: plain Python
floats, explicit loops, ``math.fsum`` for every sum, and the mask written
per element from the distance d = j - i' between key j and the aligned query
position i' = i + Sk - Sq (update notes, causal-mask change between v2.0.x and
v2.1): causal requires d <= 0; a window (left, right) requires
-left <= d <= right, -1 meaning unbounded ("FlashAttention 常用接口简单介绍",
§3.1).  Scores are scaled, softcapped with c·tanh(s/c) (update notes, v2.6),
biased with -slope·|d| (v2.4) and then passed through the textbook softmax
("optimizing-attention-flash", §3 workflow one).

Shapes use nested Python lists indexed [b][s][h][d]; keep S, D small.
"""

from __future__ import annotations

import math


def _allowed(d: int, causal: bool, left: int, right: int) -> bool:
    if causal and d > 0:
        return False
    if left != -1 and d < -left:
        return False
    if right != -1 and d > right:
        return False
    return True


def attention(q, k, v, scale=None, causal=False, window=(-1, -1), softcap=0.0, slopes=None):
    """q[b][i][h][x], k/v[b][j][g][x] as nested lists of floats.

    Returns (out[b][i][h][x], lse[b][h][i]) as nested lists; a query with no
    allowed key gets out 0 and lse -inf.
    """
    B = len(q)
    Sq, Hq, D = len(q[0]), len(q[0][0]), len(q[0][0][0])
    Sk, Hkv = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    left, right = window
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[-math.inf] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Sq):
                pos = i + Sk - Sq
                keys, vals = [], []
                for j in range(Sk):
                    d = j - pos
                    if not _allowed(d, causal, left, right):
                        continue
                    s = scale * math.fsum(q[b][i][h][x] * k[b][j][g][x] for x in range(D))
                    if softcap > 0.0:
                        s = softcap * math.tanh(s / softcap)
                    if slopes is not None:
                        s -= slopes[h] * abs(d)
                    keys.append(s)
                    vals.append(j)
                if not keys:
                    continue
                top = max(keys)
                w = [math.exp(s - top) for s in keys]
                z = math.fsum(w)
                for x in range(D):
                    out[b][i][h][x] = math.fsum(wi * v[b][j][g][x] for wi, j in zip(w, vals)) / z
                lse[b][h][i] = top + math.log(z)
    return out, lse
