"""fp64 CPU oracle for decode-shaped attention (few queries against a long key/value
sequence).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the tests and ``bench.py``'s ``cpu_baseline`` leg may use it. It shares no
code with the HIP path.

The summary of the ThunderKittens paper (groovesquid.com) names attention inference next
to the training kernels without giving its shape or formulas. The plainest reading is the
same softmax attention with Nq query rows against Nk >= 1 key/value rows; when causal,
the queries are the last Nq positions of the sequence, so query i (0-based) sees keys
j <= Nk - Nq + i (bottom-right alignment; with Nq == Nk this is the forward's mask). For
one (batch, head):

  s_ij   = scale * (q_i . k_j)
  J_i    = {0..Nk-1}, or {0..Nk-Nq+i} when causal
  O_i    = sum_{j in J_i} exp(s_ij - m_i) v_j / sum_{j in J_i} exp(s_ij - m_i)
  lse_i  = m_i + ln sum_{j in J_i} exp(s_ij - m_i)

This is the definition, computed directly; how a kernel splits the keys and merges the
pieces (through lse) is not modelled here.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_decode"]


def attention_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool = False,
                     scale: float | None = None):
    """q: [B, H, Nq, D]; k, v: [B, H, Nk, D] (float arrays). Returns (O [B,H,Nq,D],
    lse [B,H,Nq]) in float64."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("expected q [B,H,Nq,D] and k, v [B,H,Nk,D]")
    nq, nk = q.shape[2], k.shape[2]
    if causal and nq > nk:
        raise ValueError("causal decode needs Nq <= Nk")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and positive")
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        visible = np.arange(nk)[None, :] <= (nk - nq + np.arange(nq))[:, None]
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", e, v) / l
    return o, (m + np.log(l))[..., 0]
