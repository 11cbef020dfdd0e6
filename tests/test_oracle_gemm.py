"""Pins of the fp64 GEMM oracle (CPU only): pure-Python triple loops with math.fsum on
tiny shapes, an identity and a permutation, a rank-one closed form, and the shape checks."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle


def test_brute_force():
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal((5, 7)), rng.standard_normal((3, 7))
    c = oracle.gemm_nt(a, b)
    for i in range(5):
        for j in range(3):
            assert abs(c[i, j] - math.fsum(a[i, k] * b[j, k] for k in range(7))) < 1e-12


def test_identity_and_permutation():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((6, 6))
    assert np.array_equal(oracle.gemm_nt(a, np.eye(6)), a)
    perm = np.eye(6)[[3, 0, 5, 1, 4, 2]]
    # (A P^T)[:, j] = A[:, perm index of row j of P]
    assert np.array_equal(oracle.gemm_nt(a, perm), a[:, [3, 0, 5, 1, 4, 2]])


def test_rank_one():
    u, v, w = np.arange(1.0, 5.0), np.arange(2.0, 5.0), np.array([0.5, -1.0])
    a = np.outer(u, w)      # [4, 2]
    b = np.outer(v, w)      # [3, 2]
    assert np.allclose(oracle.gemm_nt(a, b), np.outer(u, v) * (w @ w), atol=1e-14)


def test_rejects_mismatched_k():
    with pytest.raises(ValueError):
        oracle.gemm_nt(np.zeros((2, 3)), np.zeros((2, 4)))
