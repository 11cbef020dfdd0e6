"""fp64 CPU oracle for the attention backward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the tests and ``bench.py``'s ``cpu_baseline`` leg may use it. It shares no
code with the HIP path.

The pages name the backward pass as a further kernel of the tile library (the summary of
the ThunderKittens paper on groovesquid.com lists attention backward among the kernels it
was used for) but give neither its formulas nor code. What it computes is therefore the
plain gradient of the forward definition in ``oracle.attention``, by the chain rule, for
one (batch, head) with incoming gradient dO of the output:

  P_ij   = exp(s_ij - lse_i) for j in J_i, 0 otherwise      (the forward's probabilities)
  dV     = P^T dO                                           (O = P V)
  dP     = dO V^T
  Delta_i = sum_j P_ij dP_ij  (= sum_d dO_id O_id)
  dS_ij  = P_ij (dP_ij - Delta_i)                           (softmax's Jacobian, row-wise)
  dQ     = scale * dS K                                     (s_ij = scale q_i . k_j)
  dK     = scale * dS^T Q

Nothing here is blocked or fused: per row chunk, matrix products, an exp and row sums.
The probabilities are recomputed from the scores and the forward's definition of lse,
not taken from any kernel. The incoming gradient of lse is taken as zero (the output
whose gradient is asked for is O).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["attention_bwd_head", "attention_bwd"]


def _probs(qc: np.ndarray, k: np.ndarray, rows: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """Softmax probabilities of the query rows ``rows`` (global indices) over all keys."""
    s = scale * (qc @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_bwd_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       causal: bool, scale: float, chunk: int = 512):
    """Gradients (dQ, dK, dV) of one head; q, k, v, do are [N, D] float64 arrays."""
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        rows = np.arange(r0, r1)
        p = _probs(q[r0:r1], k, rows, causal, scale)       # [c, N]
        doc = do[r0:r1]
        dv += p.T @ doc
        dp = doc @ v.T                                       # [c, N]
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  causal: bool = False, scale: float | None = None,
                  workers: int | None = None, chunk: int = 512):
    """Gradients over [B, H, N, D] arrays: returns (dQ, dK, dV) as float64 arrays."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape or q.shape != do.shape:
        raise ValueError("expected four [B, H, N, D] arrays of one shape")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and positive")
    b, h = q.shape[:2]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(q.shape, dtype=np.float64)
    dv = np.empty(q.shape, dtype=np.float64)

    def run(bh):
        bi, hi = bh
        dq[bi, hi], dk[bi, hi], dv[bi, hi] = attention_bwd_head(
            q[bi, hi].astype(np.float64), k[bi, hi].astype(np.float64),
            v[bi, hi].astype(np.float64), do[bi, hi].astype(np.float64), causal, scale, chunk)

    heads = [(bi, hi) for bi in range(b) for hi in range(h)]
    nw = min(workers or len(os.sched_getaffinity(0)), len(heads))
    if nw <= 1:
        for bh in heads:
            run(bh)
    else:
        with ThreadPoolExecutor(max_workers=nw) as ex:
            list(ex.map(run, heads))
    return dq, dk, dv
