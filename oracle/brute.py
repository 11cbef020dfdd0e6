"""Pure-Python brute-force attention for tiny shapes.

TEST INFRASTRUCTURE ONLY (see ``oracle/attention.py``). Written independently of the
numpy oracle: explicit loops over (i, j, d), ``math.exp`` and ``math.fsum`` (exactly
rounded sums), no numpy. It states the same definition of softmax attention and is used
to pin the numpy oracle on N <= 16, D <= 8.

Definition followed (the attention forward of the ThunderKittens pages: the warp-level
inner loop on alanwu.xyz and the H100 listing on the 10100.com review): for each query i,
  weights w_ij = exp(scale*q_i.k_j - c_i) over visible keys (j <= i if causal), with any
  finite shift c_i (here the row max), O_i = sum_j w_ij v_j / sum_j w_ij, and
  lse_i = c_i + ln sum_j w_ij.
"""
from __future__ import annotations

import math


def attention_brute(q, k, v, causal: bool, scale: float):
    """q, k: lists of N rows of D floats; v: N rows of Dv floats. Returns (O rows, lse list)."""
    n = len(q)
    o, lse = [], []
    for i in range(n):
        visible = range(i + 1) if causal else range(len(k))
        s = {j: scale * math.fsum(q[i][d] * k[j][d] for d in range(len(q[i]))) for j in visible}
        c = max(s.values())
        w = {j: math.exp(s[j] - c) for j in s}
        total = math.fsum(w.values())
        row = []
        for d in range(len(v[0])):
            row.append(math.fsum(w[j] * v[j][d] for j in w) / total)
        o.append(row)
        lse.append(c + math.log(total))
    return o, lse
