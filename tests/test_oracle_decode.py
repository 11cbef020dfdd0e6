"""Pins of the fp64 decode-shaped attention oracle (CPU only).

It is checked against the separately pinned forward oracle, which it must equal when
Nq == Nk, and whose last Nq rows of a causal problem it must reproduce (the bottom-right
alignment); against the split-and-merge identity through lse that a split-KV kernel
relies on; and against closed forms (one query, equal value rows).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_square_equals_forward(causal):
    q, k, v = (_rand((2, 3, 37, 16), s) for s in (1, 2, 3))
    o, lse = oracle.attention_decode(q, k, v, causal, 0.3)
    ro, rl = oracle.attention_fwd(q, k, v, causal, 0.3, workers=1)
    assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


@pytest.mark.parametrize("nq", [1, 3, 8])
def test_causal_rows_are_the_last_rows_of_a_square_problem(nq):
    nk, d = 50, 8
    qfull, k, v = (_rand((1, 2, nk, d), s) for s in (4, 5, 6))
    ro, rl = oracle.attention_fwd(qfull, k, v, True, 0.5, workers=1)
    o, lse = oracle.attention_decode(qfull[:, :, nk - nq:], k, v, True, 0.5)
    assert np.abs(o - ro[:, :, nk - nq:]).max() < 1e-12
    assert np.abs(lse - rl[:, :, nk - nq:]).max() < 1e-12


def test_single_query_causal_sees_every_key():
    q, k, v = _rand((1, 1, 1, 8), 7), _rand((1, 1, 40, 8), 8), _rand((1, 1, 40, 8), 9)
    a = oracle.attention_decode(q, k, v, True, 0.4)
    b = oracle.attention_decode(q, k, v, False, 0.4)
    assert np.abs(a[0] - b[0]).max() < 1e-15 and np.abs(a[1] - b[1]).max() < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_split_and_merge_through_lse(causal):
    """Keys split in two parts; each part's (O, lse) merged by weights exp(lse_s - lse)
    gives the whole. For causal parts the mask of each query is applied per part."""
    nq, nk, d, cut = 4, 70, 8, 29
    q, k, v = _rand((1, 1, nq, d), 10), _rand((1, 1, nk, d), 11), _rand((1, 1, nk, d), 12)
    o, lse = oracle.attention_decode(q, k, v, causal, 0.6)
    scale = 0.6
    parts = []
    for lo, hi in ((0, cut), (cut, nk)):
        s = scale * np.einsum("bhid,bhjd->bhij", q, k[:, :, lo:hi])
        if causal:
            vis = np.arange(lo, hi)[None, :] <= (nk - nq + np.arange(nq))[:, None]
            s = np.where(vis, s, -np.inf)
        m = s.max(-1, keepdims=True)
        e = np.exp(s - m)
        parts.append((np.einsum("bhij,bhjd->bhid", e, v[:, :, lo:hi]) / e.sum(-1, keepdims=True),
                      (m + np.log(e.sum(-1, keepdims=True)))[..., 0]))
    lse_m = np.logaddexp(parts[0][1], parts[1][1])
    o_m = sum(np.exp(l - lse_m)[..., None] * op for op, l in parts)
    assert np.abs(lse_m - lse).max() < 1e-12 and np.abs(o_m - o).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_equal_value_rows(causal):
    q, k = _rand((1, 2, 5, 8), 13), _rand((1, 2, 33, 8), 14)
    v = np.repeat(_rand((1, 2, 1, 8), 15), 33, axis=2)
    o, _ = oracle.attention_decode(q, k, v, causal, 1.0)
    assert np.abs(o - v[:, :, :5]).max() < 1e-12


def test_rejects_causal_with_more_queries_than_keys():
    with pytest.raises(ValueError):
        oracle.attention_decode(_rand((1, 1, 5, 4), 1), _rand((1, 1, 3, 4), 2), _rand((1, 1, 3, 4), 3), True)
