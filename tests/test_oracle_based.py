"""Pins of the Based linear-attention oracle (``oracle.based``) against things other than
itself: a hand-worked example, pure-Python brute force of the definition, the running-sum
(linear-time) form, closed forms, invariances, and the softmax-attention oracle, which the
Taylor weights must approach as the scores shrink (with a rigorous bound)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle.based import based_linear_attention, based_recurrent, feature_map, taylor_weight


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def brute(q, k, v):
    """Pure-Python loops over the definition: s = q.k / sqrt(d), w = 1 + s + s^2/2 for
    j <= i, o_i = sum_j w v_j / sum_j w."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, N, dv))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                ws = []
                for j in range(i + 1):
                    s = math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d)) / math.sqrt(d)
                    ws.append(1.0 + s + s * s / 2.0)
                den = math.fsum(ws)
                for c in range(dv):
                    out[b, h, i, c] = math.fsum(w * float(v[b, h, j, c]) for j, w in enumerate(ws)) / den
    return out


def test_hand_worked_example():
    # d = 1: q = (1, 2), k = (1, 0), v = (1, 3).
    # row 0: s = 1, w = 1 + 1 + 1/2 = 2.5, o = 1.
    # row 1: s_10 = 2 -> w = 1 + 2 + 2 = 5; s_11 = 0 -> w = 1; o = (5*1 + 1*3) / 6 = 4/3.
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([1.0, 0.0]).reshape(1, 1, 2, 1)
    v = np.array([1.0, 3.0]).reshape(1, 1, 2, 1)
    o = based_linear_attention(q, k, v)
    assert o[0, 0, 0, 0] == pytest.approx(1.0, abs=1e-15)
    assert o[0, 0, 1, 0] == pytest.approx(4.0 / 3.0, abs=1e-15)


@pytest.mark.parametrize("B,H,N,d,dv", [(1, 1, 1, 16, 8), (1, 2, 7, 16, 5), (2, 1, 13, 4, 3), (1, 1, 9, 9, 2)])
def test_matches_brute_force(B, H, N, d, dv):
    q, k = rand((B, H, N, d), 1), rand((B, H, N, d), 2)
    v = rand((B, H, N, dv), 3)
    np.testing.assert_allclose(based_linear_attention(q, k, v), brute(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [1, 4, 16])
def test_feature_map_inner_product_is_taylor_weight(d):
    x, y = rand((50, d), 4), rand((50, d), 5)
    fx, fy = feature_map(x), feature_map(y)
    assert fx.shape == (50, 1 + d + d * d)
    s = np.einsum("nd,nd->n", x, y) / math.sqrt(d)
    np.testing.assert_allclose(np.einsum("nf,nf->n", fx, fy), 1.0 + s + s * s / 2.0, rtol=1e-12, atol=1e-12)


def test_weights_positive():
    s = np.linspace(-50, 50, 10001)
    assert (taylor_weight(s) >= 0.5).all()
    assert taylor_weight(-1.0) == 0.5


@pytest.mark.parametrize("N", [1, 5, 64, 130])
def test_running_sum_form_equals_definition(N):
    q, k = rand((1, 2, N, 16), 6), rand((1, 2, N, 16), 7)
    v = rand((1, 2, N, 8), 8)
    np.testing.assert_allclose(based_recurrent(q, k, v), based_linear_attention(q, k, v), rtol=1e-10, atol=1e-12)


def test_zero_queries_give_prefix_means():
    # q = 0: every score is 0, every weight 1, so o_i is the mean of v_0..v_i
    N = 40
    v = rand((1, 1, N, 6), 9)
    o = based_linear_attention(np.zeros((1, 1, N, 16)), rand((1, 1, N, 16), 10), v)
    means = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], means, rtol=1e-13, atol=1e-13)


def test_zero_keys_give_prefix_means():
    N = 33
    v = rand((2, 1, N, 4), 11)
    o = based_linear_attention(rand((2, 1, N, 16), 12), np.zeros((2, 1, N, 16)), v)
    means = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(o, means, rtol=1e-13, atol=1e-13)


def test_first_row_is_first_value():
    q, k, v = rand((3, 2, 20, 16), 13), rand((3, 2, 20, 16), 14), rand((3, 2, 20, 7), 15)
    np.testing.assert_allclose(based_linear_attention(q, k, v)[:, :, 0], v[:, :, 0], rtol=0, atol=1e-14)


def test_affine_equivariance_in_v():
    q, k, v = rand((1, 2, 50, 16), 16), rand((1, 2, 50, 16), 17), rand((1, 2, 50, 5), 18)
    o = based_linear_attention(q, k, v)
    shift = np.array([1.5, -2.0, 0.25, 3.0, -0.5])
    np.testing.assert_allclose(based_linear_attention(q, k, 3.0 * v + shift), 3.0 * o + shift, rtol=1e-12, atol=1e-12)


def test_causality():
    # changing a later key or value leaves every earlier row unchanged
    q, k, v = rand((1, 1, 30, 16), 19), rand((1, 1, 30, 16), 20), rand((1, 1, 30, 4), 21)
    o = based_linear_attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 20] += 5.0
    v2[0, 0, 20] -= 7.0
    o2 = based_linear_attention(q, k2, v2)
    np.testing.assert_array_equal(o[0, 0, :20], o2[0, 0, :20])
    assert np.abs(o[0, 0, 20:] - o2[0, 0, 20:]).max() > 1e-3


@pytest.mark.parametrize("eps", [0.3, 0.15])
def test_approaches_softmax_attention_for_small_scores(eps):
    """With w_j = e^{s_j}(1 - r_j), the Based output differs from softmax attention with
    the same scale (1/sqrt(d)) and causal mask by -sum_j p_j r_j (v_j - o_soft) /
    (1 - sum_j p_j r_j), so |o_based - o_soft| <= 2 R max|v| / (1 - R) with
    R = max_j |r_j| = max |1 - (1 + s + s^2/2) e^{-s}| = O(|s|^3)."""
    N, d = 48, 16
    q, k = rand((1, 2, N, d), 22, eps), rand((1, 2, N, d), 23, eps)
    v = rand((1, 2, N, 8), 24)
    ob = based_linear_attention(q, k, v)
    os_, _ = oracle.attention_fwd(q, k, v, True, 1.0 / math.sqrt(d))
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)
    s = s[:, :, np.tril_indices(N)[0], np.tril_indices(N)[1]]
    R = float(np.abs(1.0 - taylor_weight(s) * np.exp(-s)).max())
    bound = 2.0 * R * np.abs(v).max() / (1.0 - R)
    diff = float(np.abs(ob - os_).max())
    assert diff <= bound
    # and the difference is genuinely third order: far below the first-order gap that a
    # wrong score scale would leave
    assert diff < 0.05 * float(np.abs(s).max()) ** 2
