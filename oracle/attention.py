"""fp64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP path.

What it computes is the plain definition of softmax attention, not the tiled
algorithm. The tiled online-softmax loop shown on the pages (the warp-level inner loop
on "ThunderKittens" at alanwu.xyz, and the consumer ``compute``/``finish`` steps of the
H100 attention listing on the 10100.com review, section "用TK写算子") rescales
partial sums so that, in exact arithmetic, it reaches this same result; the identity is
checked separately against ``oracle.online``.

For one (batch, head) with query rows q_i, key rows k_j, value rows v_j (all length D)
and a positive ``scale``:

  s_ij   = scale * (q_i . k_j)
  J_i    = {0..N-1}, or {0..i} when causal (lower-triangular mask, diagonal kept)
  m_i    = max_{j in J_i} s_ij
  l_i    = sum_{j in J_i} exp(s_ij - m_i)
  O_i    = sum_{j in J_i} exp(s_ij - m_i) v_j / l_i
  lse_i  = m_i + ln l_i          (natural log of sum_j exp(s_ij); not on the pages)

Readings of the pages taken here (the pages never state them):
  * lse is the natural-log logsumexp of the *scaled, masked* scores.
  * the scale is a runtime argument; the math is base e (exp2 with scale*log2(e) folded
    in is only an implementation device of the listing's TEMPERATURE_SCALE constant).
  * causal keeps j <= i, top-left aligned (queries and keys have the same length).
  * every key 0..N-1 takes part, for any N >= 1 (the warp-level loop masks the tail tile
    with -inf; the listing's integer tile count would drop a ragged tail).

Inputs are float arrays; bf16 inputs are converted exactly to float64 by the caller.
All arithmetic here is float64 numpy: a matrix product per row chunk, a row max, exp,
a row sum, and a second matrix product.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "attention_head",
    "attention_fwd",
    "attention_rows",
    "attention_probs",
]


def _check(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> None:
    if q.ndim != k.ndim or q.ndim != v.ndim:
        raise ValueError("q, k, v must have the same rank")
    if q.shape[-1] != k.shape[-1]:
        raise ValueError("q and k must share the head dimension D")
    if k.shape[-2] != v.shape[-2]:
        raise ValueError("k and v must have the same number of rows")
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and positive")


def _scores(qc: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = scale * q_i . k_j for a block of query rows (fp64)."""
    return scale * (qc @ k.T)


def _allowed(i0: int, i1: int, nk: int, causal: bool) -> np.ndarray:
    """Boolean [i1-i0, nk]: key j is visible to query i (j <= i when causal)."""
    if not causal:
        return np.ones((i1 - i0, nk), dtype=bool)
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(nk)[None, :]
    return cols <= rows


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                   scale: float, chunk: int = 512) -> tuple[np.ndarray, np.ndarray]:
    """Attention for one head. q: [N, D], k: [N, D], v: [N, Dv]. Returns (O [N, Dv], lse [N])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v, scale)
    n = q.shape[0]
    if causal and k.shape[0] != n:
        raise ValueError("causal attention needs as many keys as queries")
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for i0 in range(0, n, chunk):
        i1 = min(n, i0 + chunk)
        kend = i1 if causal else k.shape[0]  # keys beyond the chunk's last row are all masked
        s = _scores(q[i0:i1], k[:kend], scale)
        s = np.where(_allowed(i0, i1, kend, causal), s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        o[i0:i1] = (e @ v[:kend]) / l[:, None]
        lse[i0:i1] = m + np.log(l)
    return o, lse


def _workers(requested: int | None) -> int:
    if requested is not None:
        return max(1, int(requested))
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool = False,
                  scale: float | None = None, workers: int | None = None,
                  chunk: int = 512) -> tuple[np.ndarray, np.ndarray]:
    """Attention over [B, H, N, D] arrays. Returns (O [B,H,N,D] fp64, lse [B,H,N] fp64).

    Heads are independent; they are spread over ``workers`` threads (numpy releases the
    GIL inside its matrix products and elementwise kernels).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, D] arrays")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    _check(q, k, v, scale)
    b, h, n, _ = q.shape
    o = np.empty(q.shape[:3] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty((b, h, n), dtype=np.float64)
    heads = [(bi, hi) for bi in range(b) for hi in range(h)]

    def run(bh):
        bi, hi = bh
        o[bi, hi], lse[bi, hi] = attention_head(q[bi, hi], k[bi, hi], v[bi, hi], causal, scale, chunk)

    nw = min(_workers(workers), len(heads))
    if nw <= 1:
        for bh in heads:
            run(bh)
    else:
        with ThreadPoolExecutor(max_workers=nw) as ex:
            list(ex.map(run, heads))
    return o, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, causal: bool = False,
                   scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """O and lse for selected output rows only, each computed on its own.

    ``rows`` is a sequence of (b, h, i). Returns (O [R, D] fp64, lse [R] fp64). Used at
    sizes where the full oracle would take too long: each row costs one pass over K, V.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    _check(q, k, v, scale)
    rows = list(rows)
    o = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for r, (bi, hi, i) in enumerate(rows):
        kend = i + 1 if causal else k.shape[2]
        qi = np.asarray(q[bi, hi, i], dtype=np.float64)
        kk = np.asarray(k[bi, hi, :kend], dtype=np.float64)
        vv = np.asarray(v[bi, hi, :kend], dtype=np.float64)
        s = scale * (kk @ qi)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[r] = (e @ vv) / l
        lse[r] = m + math.log(l)
    return o, lse


def attention_probs(q: np.ndarray, k: np.ndarray, causal: bool = False,
                    scale: float | None = None) -> np.ndarray:
    """The full probability matrix P [N, N] of one head (small shapes only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    n = q.shape[0]
    s = _scores(q, k, scale)
    s = np.where(_allowed(0, n, k.shape[0], causal), s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return e / e.sum(axis=1)[:, None]
