"""fp64 CPU oracle for the plain matrix product on the tile layer.

TEST INFRASTRUCTURE ONLY. Only the tests and ``bench.py``'s ``cpu_baseline`` leg may
use it; it shares no code with the HIP path.

The tile library's pages show its matrix-multiply building blocks (the warp-level
``mma`` and the warpgroup ``mm_ABt`` / ``mma_AB`` calls of the attention listing) and the
paper summary names GEMM among its kernels. The product computed here is the plain
definition C = A B^T with A [M, K] and B [N, K] (both row-major, K contiguous: the
layout of ``mm_ABt``), C[i, j] = sum_k A[i, k] B[j, k], in float64.
"""
from __future__ import annotations

import numpy as np

__all__ = ["gemm_nt"]


def gemm_nt(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = A @ B^T in float64; a is [M, K], b is [N, K]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("expected a [M, K] and b [N, K]")
    return a @ b.T
