"""The tiled online-softmax recurrence, in float64, with arbitrary tile sizes.

TEST INFRASTRUCTURE ONLY (see ``oracle/attention.py``). This is the method's own
algorithm, used to pin that it reaches the plain definition: tests run it with random
(query-tile, key-tile) sizes and compare it with ``oracle.attention`` to ~1e-12.

Steps, in the order the pages give them (warp-level inner loop on the "ThunderKittens"
blog at alanwu.xyz; consumer ``setup``/``compute``/``finish`` of the H100 attention
listing in the 10100.com review, section "用TK写算子"):

  setup:   O = 0, l = 0, m = -inf for every query row of the tile
  per key tile:
    S      = Q_tile K_tile^T                      (raw scores)
    mask   keys past the end (and, causal, keys after the query) set to -inf
    m_new  = max(m, rowmax S)                     (running max of raw scores)
    P      = exp2(c*S - c*m_new)                  (c = scale*log2 e, the listing's
                                                   TEMPERATURE_SCALE with a runtime scale)
    alpha  = exp2(c*m - c*m_new)                  (rescale factor of earlier tiles)
    l      = alpha*l + rowsum P
    O      = alpha*O + P V_tile
    m      = m_new
  finish:  O = O / l ; lse = (c*m + log2 l) * ln 2   (lse is not on the pages; natural log)

In exact arithmetic this telescopes to the definition. Tiles are visited in ascending key
order, so the first tile holds key 0, which every query sees: m is finite from then on.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def attention_online(q, k, v, causal: bool, scale: float, br: int, bc: int):
    """One head. q, k: [N, D]; v: [N, Dv]. Returns (O [N, Dv], lse [N]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, nk = q.shape[0], k.shape[0]
    c = scale * LOG2E
    o_all = np.empty((n, v.shape[1]))
    lse_all = np.empty(n)
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        rows = np.arange(i0, i1)
        o = np.zeros((i1 - i0, v.shape[1]))
        l = np.zeros(i1 - i0)
        m = np.full(i1 - i0, -np.inf)
        for j0 in range(0, nk, bc):
            if causal and j0 > i1 - 1:
                break  # every key of this tile and later ones is after every query here
            j1 = min(nk, j0 + bc)
            s = q[i0:i1] @ k[j0:j1].T
            cols = np.arange(j0, j1)
            if causal:
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            p = np.exp2(c * s - (c * m_new)[:, None])
            alpha = np.exp2(c * m - c * m_new)
            l = alpha * l + p.sum(axis=1)
            o = alpha[:, None] * o + p @ v[j0:j1]
            m = m_new
        o_all[i0:i1] = o / l[:, None]
        lse_all[i0:i1] = (c * m + np.log2(l)) * math.log(2.0)
    return o_all, lse_all
