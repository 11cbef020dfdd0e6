"""Pins of the fp64 backward oracle (CPU only).

The backward oracle is checked against things it does not compute itself:
  * central finite differences of L = sum(O * dO), with O from the (separately pinned)
    forward oracle, for every entry of dQ, dK and dV on tiny shapes;
  * invariants that follow from the softmax: the key-sum of dK is zero, the key-sum of
    dV equals the query-sum of dO, equal value rows give zero dQ and dK, one key gives
    dQ = dK = 0 and dV = dO;
  * planted mistakes (no Delta term, missing scale, transposed dS, P in place of dS) fail
    the finite-difference pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle.backward import _probs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.attention_fwd(q[None, None], k[None, None], v[None, None], causal, scale, workers=1)
    return float((o[0, 0] * do).sum())


def _finite_diff(q, k, v, do, causal, scale, h=1e-6):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (_loss(*plus, do, causal, scale) - _loss(*minus, do, causal, scale)) / (2 * h)
        grads.append(g)
    return grads


def _inputs(n, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, d)), rng.standard_normal((n, d)),
            rng.standard_normal((n, d)), rng.standard_normal((n, d)))


CASES = [(1, 3, False), (2, 3, True), (5, 4, False), (5, 4, True), (8, 3, True), (9, 2, False)]


@pytest.mark.parametrize("n,d,causal", CASES)
def test_matches_finite_differences(n, d, causal):
    q, k, v, do = _inputs(n, d, seed=10 * n + d + causal)
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd_head(q, k, v, do, causal, scale)
    fq, fk, fv = _finite_diff(q, k, v, do, causal, scale)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(got - want).max() <= 1e-6 * max(1.0, np.abs(want).max())


def test_full_tensor_api_matches_per_head():
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((2, 3, 40, 8)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, 0.3, workers=2, chunk=16)
        for b in range(2):
            for h in range(3):
                hq, hk, hv = oracle.attention_bwd_head(q[b, h], k[b, h], v[b, h], do[b, h], causal, 0.3)
                assert np.allclose(dq[b, h], hq, atol=1e-12)
                assert np.allclose(dk[b, h], hk, atol=1e-12)
                assert np.allclose(dv[b, h], hv, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    q, k, v, do = _inputs(64, 16, seed=5)
    dq, dk, dv = oracle.attention_bwd_head(q, k, v, do, causal, 0.25, chunk=20)
    # each row of dS sums to zero over its visible keys, so dK sums to zero over keys
    assert np.abs(dk.sum(axis=0)).max() < 1e-10
    # each row of P sums to one, so the key-sum of dV is the query-sum of dO
    assert np.abs(dv.sum(axis=0) - do.sum(axis=0)).max() < 1e-10


@pytest.mark.parametrize("causal", [False, True])
def test_equal_value_rows_give_zero_dq_dk(causal):
    q, k, v, do = _inputs(33, 8, seed=6)
    v = np.repeat(v[:1], 33, axis=0)
    dq, dk, dv = oracle.attention_bwd_head(q, k, v, do, causal, 0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


def test_single_key():
    q, k, v, do = _inputs(1, 8, seed=7)
    dq, dk, dv = oracle.attention_bwd_head(q, k, v, do, False, 0.5)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    assert np.array_equal(dv, do)


def test_causal_row0_gradients():
    """Row 0 sees only key 0: its probability is 1, so it adds nothing to dQ_0 and puts
    dO_0 into dV_0 whole."""
    q, k, v, do = _inputs(6, 4, seed=8)
    dq, _, dv = oracle.attention_bwd_head(q, k, v, do, True, 0.9)
    assert np.abs(dq[0]).max() < 1e-15
    p = _probs(q, k, np.arange(6), True, 0.9)
    assert np.allclose(dv[0], (p[:, 0:1] * do).sum(axis=0), atol=1e-14)


# ---------------------------------------------------------------- planted mistakes

def _mutant(q, k, v, do, causal, scale, kind):
    p = _probs(q, k, np.arange(q.shape[0]), causal, scale)
    dp = do @ v.T
    delta = (p * dp).sum(axis=1, keepdims=True)
    if kind == "no_delta":
        ds = p * dp
    elif kind == "p_not_ds":
        ds = p
    else:
        ds = p * (dp - delta)
    dq = (1.0 if kind == "no_scale" else scale) * (ds @ k)
    dk = scale * ((ds if kind == "transposed" else ds.T) @ q)
    return dq, dk, p.T @ do


@pytest.mark.parametrize("kind", ["no_delta", "p_not_ds", "no_scale", "transposed"])
def test_finite_differences_catch_planted_mistakes(kind):
    q, k, v, do = _inputs(5, 3, seed=11)
    scale = 0.7
    fq, fk, _ = _finite_diff(q, k, v, do, False, scale)
    mq, mk, _ = _mutant(q, k, v, do, False, scale, kind)
    err = max(np.abs(mq - fq).max(), np.abs(mk - fk).max())
    assert err > 1e-3, f"mutant {kind} not caught ({err})"
