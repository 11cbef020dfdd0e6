"""fp64 CPU oracle for Based linear attention (forward, causal).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the tests and ``bench.py``'s ``cpu_baseline`` leg may use it. It shares no
code with the HIP path.

The pages only name the kernel: "ThunderKittens 2.0: Faster Kernels, Talking Models, and
More Adorable Kittens" (thebeat.tech), sections "New Kernels for Enhanced Performance" and
"Performance Benchmarks", list Based linear attention among the new linear-attention
kernels with its speedup, and give neither its formulas nor its shapes. The reading taken
here is the published Based design: causal linear attention whose feature map is the
second-order Taylor expansion of exp(q.k / sqrt(d)) on d = 16 query/key features, with
the usual linear-attention normaliser. For one (batch, head), query rows q_i, key rows k_j
(length d) and value rows v_j (length dv):

  s_ij = (q_i . k_j) / sqrt(d)
  w_ij = 1 + s_ij + s_ij^2 / 2          for j <= i (causal), else 0
  o_i  = sum_j w_ij v_j / sum_j w_ij

w_ij = ((1 + s_ij)^2 + 1) / 2 >= 1/2, so the normaliser never vanishes. The same weights
are the inner product phi(q_i) . phi(k_j) of the feature map

  phi(x) = [1, x / d^(1/4), vec(x x^T) / (sqrt(2) sqrt(d))]      (1 + d + d^2 features)

which is what makes the method linear in N: o_i = phi(q_i)^T S_i / phi(q_i)^T z_i with the
running sums S_i = sum_{j<=i} phi(k_j) v_j^T and z_i = sum_{j<=i} phi(k_j). This module
computes the definition directly (the quadratic form), in row chunks; ``feature_map`` and
``based_recurrent`` (the running-sum form, for small shapes) exist so that the tests can
pin the two forms against each other.
"""
from __future__ import annotations

import numpy as np

__all__ = ["based_linear_attention", "based_recurrent", "feature_map", "taylor_weight"]


def taylor_weight(s):
    """1 + s + s^2 / 2, the second-order Taylor polynomial of exp(s)."""
    s = np.asarray(s, dtype=np.float64)
    return 1.0 + s + 0.5 * s * s


def feature_map(x: np.ndarray) -> np.ndarray:
    """phi(x) for rows x of length d: [1, x / d^(1/4), vec(x x^T) / (sqrt(2) sqrt(d))]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    quad = (x[..., :, None] * x[..., None, :]).reshape(*x.shape[:-1], d * d)
    ones = np.ones(x.shape[:-1] + (1,))
    return np.concatenate([ones, x / d ** 0.25, quad / (np.sqrt(2.0) * np.sqrt(d))], axis=-1)


def _check(q, k, v):
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if q.ndim != 4 or q.shape != k.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B,H,N,d] and v [B,H,N,dv]")
    return q, k, v


def based_linear_attention(q, k, v, row_chunk: int = 512) -> np.ndarray:
    """q, k: [B, H, N, d]; v: [B, H, N, dv] (float arrays). Returns o [B, H, N, dv] in
    float64, by the definition (causal quadratic form)."""
    q, k, v = _check(q, k, v)
    B, H, N, d = q.shape
    out = np.empty(v.shape, dtype=np.float64)
    inv = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_chunk):
                r1 = min(N, r0 + row_chunk)
                s = (q[b, h, r0:r1] @ k[b, h, :r1].T) * inv
                w = taylor_weight(s)
                w[np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]] = 0.0
                out[b, h, r0:r1] = (w @ v[b, h, :r1]) / w.sum(axis=1, keepdims=True)
    return out


def based_recurrent(q, k, v) -> np.ndarray:
    """The running-sum form: S_i = S_{i-1} + phi(k_i) v_i^T, z_i = z_{i-1} + phi(k_i),
    o_i = phi(q_i)^T S_i / phi(q_i)^T z_i. float64; memory O(d^2 dv) per head."""
    q, k, v = _check(q, k, v)
    B, H, N, _ = q.shape
    out = np.empty(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            fq = feature_map(q[b, h])
            fk = feature_map(k[b, h])
            S = np.zeros((fk.shape[1], v.shape[3]))
            z = np.zeros(fk.shape[1])
            for i in range(N):
                S += np.outer(fk[i], v[b, h, i])
                z += fk[i]
                out[b, h, i] = (fq[i] @ S) / (fq[i] @ z)
    return out
