"""The online-softmax recurrence in fp64 -- TEST INFRASTRUCTURE.

This is not the oracle's definition of attention (that is the plain batched
softmax in ``oracle.c``).  It restates the recurrence that the method rests on,
so a test can show it reaches the batched result for any block sizes:

  "Flash Attention" (aarnphm.xyz), section Deriving the online softmax, tile form:
      m_new = max(m_old, max_j S_ij)
      l_new = exp(m_old - m_new) l_old + sum_j exp(S_ij - m_new)
      O_new = exp(m_old - m_new) O_old + sum_j exp(S_ij - m_new) V_j
  with one normalisation O = O_new / l_new after the last key tile, and the
  pair (m, l) merged as a commutative monoid
      [m_a, l_a] + [m_b, l_b] = [max, l_a e^{m_a - max} + l_b e^{m_b - max}],
  identity [-inf, 0].  "Flash attention, f32", sections The loop over keys,
  Online softmax and After the loop, walk the same steps per query block.

Blocks of queries (BR rows) are independent; blocks of keys (BC keys) are
visited in order.  A key masked by causality is left out of its tile (the
tile's maximum is over live keys only), so no finite stand-in for -inf enters.
"""
from __future__ import annotations

import numpy as np


def tiled_forward(q, k, v, scale, causal=False, br=16, bc=16):
    """q [Nq,D], k/v [Nk,D] float64.  Returns (o [Nq,D], lse [Nq])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    nq, d = q.shape
    nk = k.shape[0]
    o = np.empty((nq, d))
    lse = np.empty(nq)
    for r0 in range(0, nq, br):
        rows = np.arange(r0, min(r0 + br, nq))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, d))
        for c0 in range(0, nk, bc):
            cols = np.arange(c0, min(c0 + bc, nk))
            s = scale * (q[rows] @ k[cols].T)
            live = np.ones_like(s, dtype=bool)
            if causal:
                live = cols[None, :] <= rows[:, None]
            s_live = np.where(live, s, -np.inf)
            m_tile = s_live.max(axis=1)
            m_new = np.maximum(m, m_tile)
            # rows with no live key so far keep the identity (-inf, 0, 0)
            seen = np.isfinite(m_new)
            safe = np.where(seen, m_new, 0.0)
            corr = np.where(seen, np.exp(m - safe), 1.0)
            p = np.where(live, np.exp(s - safe[:, None]), 0.0)
            l = corr * l + p.sum(axis=1)
            acc = corr[:, None] * acc + p @ v[cols]
            m = m_new
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


def partial_state(s, vals):
    """The (m, l, O) summary of one group of keys.  s [n] scores, vals [n,D]."""
    s = np.asarray(s, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    if s.size == 0:
        return -np.inf, 0.0, np.zeros(vals.shape[1])
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ vals


def merge(a, b):
    """Monoid product of two (m, l, O) summaries; identity is (-inf, 0, 0)."""
    ma, la, oa = a
    mb, lb, ob = b
    m = max(ma, mb)
    if m == -np.inf:
        return -np.inf, 0.0, np.zeros_like(oa)
    wa = 0.0 if ma == -np.inf else np.exp(ma - m)
    wb = 0.0 if mb == -np.inf else np.exp(mb - m)
    return m, la * wa + lb * wb, oa * wa + ob * wb
