"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

The pages print no attention values, so every pin comes from mathematics: a hand-derived
worked example (tests/golden), closed forms, invariants, brute force on tiny inputs, and
the pages' own tiled online-softmax recurrence (which must reach the definition). The
mutation test at the end plants plausible mistakes in the oracle and checks that some pin
fails for each of them.
"""
from __future__ import annotations

import ast
import json
import math
import operator
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oracle_attention
from softmax_attention_fwd_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_n3_d2.json")


# ----------------------------------------------------------------------------- helpers

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.Pow: operator.pow}
_FUNCS = {"ln": math.log, "exp": math.exp, "sqrt": math.sqrt}


def closed_form(expr: str) -> float:
    """Evaluate a fixture expression: numbers, e, + - * / **, ln/exp/sqrt (nothing else)."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.Name) and node.id == "e":
            return math.e
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id in _FUNCS and len(node.args) == 1):
            return _FUNCS[node.func.id](ev(node.args[0]))
        raise ValueError(f"unsupported expression: {expr}")
    return ev(ast.parse(expr, mode="eval"))


def rand_head(rng, n, d, sigma=1.0, dv=None):
    dv = d if dv is None else dv
    return (rng.standard_normal((n, d)) * sigma, rng.standard_normal((n, d)) * sigma,
            rng.standard_normal((n, dv)))


def head(q, k, v, causal, scale):
    """Run the 4-D oracle on one head (so the pins exercise attention_fwd itself)."""
    o, lse = oracle.attention_fwd(q[None, None], k[None, None], v[None, None], causal, scale,
                                  workers=1, chunk=5)
    return o[0, 0], lse[0, 0]


# ----------------------------------------------------------------------------- pins
# Each pin raises AssertionError on a mismatch; the mutation test reuses them.

def pin_golden():
    fx = json.load(open(GOLDEN))
    q, k, v = (np.array(fx[n], dtype=np.float64) for n in ("q", "k", "v"))
    for case in fx["cases"]:
        scale = closed_form(case["scale"])
        want_o = np.array([[closed_form(x) for x in row] for row in case["o"]])
        want_lse = np.array([closed_form(x) for x in case["lse"]])
        o, lse = head(q, k, v, case["causal"], scale)
        np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-14)
        # the brute force is pinned by the same hand-derived values
        bo, blse = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), case["causal"], scale)
        np.testing.assert_allclose(np.array(bo), want_o, rtol=0, atol=1e-14)
        np.testing.assert_allclose(np.array(blse), want_lse, rtol=0, atol=1e-14)


def pin_brute_force(seed=0, trials=40):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 17))
        d = int(rng.integers(1, 9))
        dv = int(rng.integers(1, 9))
        causal = bool(t % 2)
        scale = float(rng.uniform(0.05, 3.0))
        q, k, v = rand_head(rng, n, d, sigma=1.5, dv=dv)
        o, lse = head(q, k, v, causal, scale)
        bo, blse = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), causal, scale)
        np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(blse), rtol=0, atol=1e-12)


def pin_equal_v_rows(seed=1):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        q, k, _ = rand_head(rng, 13, 6, sigma=2.0)
        row = rng.standard_normal(5)
        v = np.tile(row, (13, 1))
        o, _ = head(q, k, v, causal, 0.7)
        np.testing.assert_allclose(o, np.tile(row, (13, 1)), rtol=0, atol=1e-13)


def pin_rows_sum_to_one(seed=2):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        n = 11
        q, k, _ = rand_head(rng, n, n, sigma=1.3)
        p = oracle.attention_probs(q, k, causal, 0.6)
        np.testing.assert_allclose(p.sum(axis=1), np.ones(n), rtol=0, atol=1e-12)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)
        # V = identity (N = D) reads P out through the full oracle
        o, _ = head(q, k, np.eye(n), causal, 0.6)
        np.testing.assert_allclose(o, p, rtol=0, atol=1e-13)


def pin_causal_row0(seed=3):
    rng = np.random.default_rng(seed)
    q, k, v = rand_head(rng, 9, 7, sigma=2.0)
    o, lse = head(q, k, v, True, 0.9)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - 0.9 * math.fsum(q[0, d] * k[0, d] for d in range(7))) < 1e-13


def pin_zero_query(seed=4):
    """Q = 0 (or K = 0): every visible key has weight 1/|J_i|."""
    rng = np.random.default_rng(seed)
    n, d = 10, 4
    _, k, v = rand_head(rng, n, d)
    for zero_k in (False, True):
        q = np.zeros((n, d)) if not zero_k else rng.standard_normal((n, d))
        kk = k if not zero_k else np.zeros((n, d))
        o, lse = head(q, kk, v, False, 1.1)
        np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.full(n, math.log(n)), rtol=0, atol=1e-13)
        o, lse = head(q, kk, v, True, 1.1)
        want = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
        np.testing.assert_allclose(o, want, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)


def pin_two_keys_logistic(seed=5):
    """N = 2 keys, non-causal: weight of key 0 is the logistic sigmoid of s_0 - s_1."""
    rng = np.random.default_rng(seed)
    q, k, v = rand_head(rng, 2, 3, sigma=2.0)
    scale = 0.8
    o, lse = head(q, k, v, False, scale)
    for i in range(2):
        s0 = scale * math.fsum(q[i, d] * k[0, d] for d in range(3))
        s1 = scale * math.fsum(q[i, d] * k[1, d] for d in range(3))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(o[i], w0 * v[0] + (1 - w0) * v[1], rtol=0, atol=1e-13)
        big, small = max(s0, s1), min(s0, s1)
        assert abs(lse[i] - (big + math.log1p(math.exp(small - big)))) < 1e-13


def pin_permutation_invariance(seed=6):
    rng = np.random.default_rng(seed)
    q, k, v = rand_head(rng, 12, 5)
    perm = rng.permutation(12)
    o, lse = head(q, k, v, False, 0.5)
    o2, lse2 = head(q, k[perm], v[perm], False, 0.5)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def pin_key_shift(seed=7):
    """k_j -> k_j + u: O unchanged, lse_i shifted by scale * q_i . u."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        q, k, v = rand_head(rng, 12, 5)
        u = rng.standard_normal(5)
        scale = 0.45
        o, lse = head(q, k, v, causal, scale)
        o2, lse2 = head(q, k + u, v, causal, scale)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2 - lse, scale * (q @ u), rtol=0, atol=1e-12)


def pin_single_key(seed=8):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        q, k, v = rand_head(rng, 1, 6)
        o, lse = head(q, k, v, causal, 0.3)
        np.testing.assert_array_equal(o, v)
        assert abs(lse[0] - 0.3 * math.fsum(q[0, d] * k[0, d] for d in range(6))) < 1e-14


def pin_large_scale_argmax(seed=9):
    """As scale grows, each row's weight concentrates on its largest score."""
    rng = np.random.default_rng(seed)
    q, k, v = rand_head(rng, 8, 4)
    for causal in (False, True):
        o, _ = head(q, k, v, causal, 1e4)
        s = q @ k.T
        if causal:
            s = np.where(np.tril(np.ones_like(s)) > 0, s, -np.inf)
        np.testing.assert_allclose(o, v[np.argmax(s, axis=1)], rtol=0, atol=1e-9)


def pin_online_recurrence(seed=10):
    """The pages' tiled recurrence reaches the definition for any tile sizes."""
    rng = np.random.default_rng(seed)
    for t in range(12):
        n = int(rng.integers(1, 90))
        d = int(rng.integers(1, 17))
        causal = bool(t % 2)
        scale = float(rng.uniform(0.1, 2.0))
        q, k, v = rand_head(rng, n, d, sigma=2.0)
        br, bc = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        o, lse = head(q, k, v, causal, scale)
        o2, lse2 = oracle.attention_online(q, k, v, causal, scale, br, bc)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def pin_rows_match_full(seed=11):
    """The per-row oracle used at full sizes agrees with the full-tensor oracle."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        q = rng.standard_normal((2, 3, 37, 8))
        k = rng.standard_normal((2, 3, 37, 8))
        v = rng.standard_normal((2, 3, 37, 8))
        o, lse = oracle.attention_fwd(q, k, v, causal, 0.4, workers=2, chunk=16)
        rows = [(b, h, i) for b in range(2) for h in range(3) for i in (0, 1, 15, 16, 36)]
        ro, rlse = oracle.attention_rows(q, k, v, rows, causal, 0.4)
        for r, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(ro[r], o[b, h, i], rtol=0, atol=1e-13)
            assert abs(rlse[r] - lse[b, h, i]) < 1e-13


PINS = [pin_golden, pin_brute_force, pin_equal_v_rows, pin_rows_sum_to_one, pin_causal_row0,
        pin_zero_query, pin_two_keys_logistic, pin_permutation_invariance, pin_key_shift,
        pin_single_key, pin_large_scale_argmax, pin_online_recurrence, pin_rows_match_full]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------- mutation test

def _bad_scores_no_scale(qc, k, scale):
    return qc @ k.T


def _bad_scores_sign(qc, k, scale):
    return -scale * (qc @ k.T)


def _bad_allowed_strict(i0, i1, nk, causal):
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(nk)[None, :]
    return (cols < rows) | (cols == 0) if causal else np.ones((i1 - i0, nk), bool)


def _bad_allowed_upper(i0, i1, nk, causal):
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(nk)[None, :]
    return (cols >= rows) | (rows == nk - 1) if causal else np.ones((i1 - i0, nk), bool)


def _bad_allowed_offset(i0, i1, nk, causal):
    # forgets the chunk offset: row index restarts at 0 in every chunk
    rows = np.arange(0, i1 - i0)[:, None]
    cols = np.arange(nk)[None, :]
    return cols <= rows if causal else np.ones((i1 - i0, nk), bool)


MUTANTS = {
    "scale dropped": ("_scores", _bad_scores_no_scale),
    "score sign flipped": ("_scores", _bad_scores_sign),
    "causal mask drops diagonal": ("_allowed", _bad_allowed_strict),
    "causal mask upper triangle": ("_allowed", _bad_allowed_upper),
    "causal mask ignores chunk offset": ("_allowed", _bad_allowed_offset),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(oracle_attention, attr, bad)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin fails when the oracle has the mistake: {name}"


def test_mutant_lse_log2_is_caught(monkeypatch):
    """lse in base 2 instead of natural log must fail a pin."""
    real = oracle_attention.attention_head

    def bad(q, k, v, causal, scale, chunk=512):
        o, lse = real(q, k, v, causal, scale, chunk)
        return o, lse / math.log(2.0)
    monkeypatch.setattr(oracle_attention, "attention_head", bad)
    with pytest.raises(AssertionError):
        pin_golden()


def test_mutant_q_k_swapped_is_caught(monkeypatch):
    """A transposed score matrix (s_ij = q_j . k_i, i.e. Q and K swapped) must fail a pin."""
    real = oracle_attention.attention_head

    def bad(q, k, v, causal, scale, chunk=512):
        return real(k, q, v, causal, scale, chunk)
    monkeypatch.setattr(oracle_attention, "attention_head", bad)
    with pytest.raises(AssertionError):
        pin_golden()
    with pytest.raises(AssertionError):
        pin_brute_force()


def test_mutant_value_rows_shifted_is_caught(monkeypatch):
    """Pairing weight j with v_{j+1} (an index slip) must fail a pin."""
    real = oracle_attention.attention_head

    def bad(q, k, v, causal, scale, chunk=512):
        return real(q, k, np.roll(np.asarray(v), 1, axis=0), causal, scale, chunk)
    monkeypatch.setattr(oracle_attention, "attention_head", bad)
    failures = 0
    for pin in (pin_golden, pin_causal_row0, pin_brute_force):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 2


# ----------------------------------------------------------------------------- input recipe

def test_inputs_deterministic_and_bf16():
    a = inputs.make_qkv(2, 3, 17, 8, seed=5)
    b = inputs.make_qkv(2, 3, 17, 8, seed=5)
    c = inputs.make_qkv(2, 3, 17, 8, seed=6)
    import torch
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape == (2, 3, 17, 8)
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a[0], c[0])


def test_inputs_sigma_and_rounding():
    import torch
    q, k, v = inputs.make_qkv(1, 2, 4096, 16, seed=9, sigma_q=2.0, sigma_k=2.0, sigma_v=1.0)
    assert abs(q.float().std().item() - 2.0) < 0.05
    assert abs(v.float().std().item() - 1.0) < 0.03
    # the recipe rounds float32 draws to bf16 with round-to-nearest-even
    g = torch.Generator().manual_seed(9)
    x = torch.randn((1, 2, 4096, 16), generator=g) * 2.0
    bits = x.view(torch.int32)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).to(torch.int16)
    assert torch.equal(q.view(torch.int16), rne)


def test_workload_table():
    w = inputs.WORKLOADS
    assert [(x.B, x.H, x.N, x.D, x.causal) for x in w.values()] == [
        (1, 1, 128, 64, False), (16, 16, 1024, 64, False), (16, 16, 4096, 128, False),
        (8, 32, 8192, 128, True), (1, 32, 16384, 128, True)]
    assert w[5].sigma_q == 2.0 and w[5].sigma_k == 2.0 and w[5].sigma_v == 1.0
    assert abs(w[3].flops - 2.199023255552e12) < 1e3
    assert w[4].flops == 4.0 * 8 * 32 * 8192 ** 2 * 128 / 2
