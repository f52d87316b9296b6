"""Pure-Python brute-force attention for tiny inputs -- TEST INFRASTRUCTURE.

Written straight from the definition of softmax ("Flash Attention" (aarnphm.xyz),
Definition 1): softmax(z)_i = e^{z_i} / sum_j e^{z_j}, with no maximum
subtracted, and O = softmax(scale Q K^T) V ("Flash attention, f32", opening
paragraph).  Sums use ``math.fsum`` so they are correctly rounded.  Causal keeps
key j for query i only when j <= i ("06: Fused attention", attn_fwd).

Because nothing is shifted, it is valid only while |scale * q.k| stays far below
exp's overflow (about 709 in fp64); callers keep scores under 30.
It exists to pin the C oracle: the two share no code.
"""
from __future__ import annotations

import math


def attention(q, k, v, scale, causal=False):
    """q: Nq lists of D floats; k, v: Nk lists of D floats.

    Returns (o, lse): o is Nq lists of D floats, lse is Nq floats (natural log of
    the sum of exponentials of the scaled scores).
    """
    nq, nk = len(q), len(k)
    d = len(q[0])
    out, lse = [], []
    for i in range(nq):
        keys = range(i + 1) if causal else range(nk)
        weights = []
        for j in keys:
            score = scale * math.fsum(q[i][t] * k[j][t] for t in range(d))
            weights.append((j, math.exp(score)))
        z = math.fsum(w for _, w in weights)
        row = [math.fsum(w * v[j][t] for j, w in weights) / z for t in range(d)]
        out.append(row)
        lse.append(math.log(z))
    return out, lse
