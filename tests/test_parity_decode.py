"""GPU parity of the decode-shaped attention (split-KV, merged through lse; through the
C ABI) against the fp64 decode oracle, with the forward's bar (the arithmetic is the
forward's plus an fp32 merge of the chunks): O max-abs <= 2e-2, rel-L2 <= 5e-3, lse
max-abs <= 1e-3, over every element.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_fwd_amd import attn_decode, attn_fwd, decode_workspace_bytes
from softmax_attention_fwd_amd.inputs import DECODE_WORKLOADS, decode_inputs, make_qkv

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check(o, lse, o_ref, lse_ref, what):
    og, lg = f64(o), f64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), f"{what}: non-finite output"
    d = og - o_ref
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / np.linalg.norm(o_ref))
    lse_err = float(np.abs(lg - lse_ref).max())
    print(f"[parity-decode] {what}: O max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse max-abs {lse_err:.3e}",
          flush=True)
    assert max_abs <= O_MAX_ABS and rel <= O_REL_L2 and lse_err <= LSE_MAX_ABS, what


def run(q, k, v, causal, scale):
    dev = torch.device("cuda:0")
    o, lse = attn_decode(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def rand(shape, seed, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(torch.bfloat16)


SHAPES = [
    # B, H, Nq, Nk, D, causal, sigma_qk
    (1, 1, 1, 1, 64, False, 1.0), (1, 1, 1, 1, 128, True, 1.0),
    (1, 2, 1, 100, 128, True, 1.0), (1, 1, 1, 33, 128, False, 1.0),
    (2, 2, 4, 257, 64, False, 1.0), (2, 2, 4, 257, 64, True, 1.0),
    (1, 1, 5, 130, 128, True, 1.0), (1, 3, 8, 1000, 128, True, 1.0),
    (2, 1, 16, 4096, 128, False, 1.0), (1, 2, 32, 2048, 64, True, 1.0),
    (1, 2, 32, 32, 128, True, 1.0), (1, 2, 7, 5000, 128, True, 2.0),
    (3, 1, 2, 300, 64, False, 2.0),
    # more heads than compute units (little or no split), and one head whose ragged cache
    # is split over the most workgroups
    (16, 32, 1, 512, 128, True, 1.0), (1, 1, 1, 65537, 64, False, 1.0),
]


@pytest.mark.parametrize("B,H,Nq,Nk,D,causal,sigma", SHAPES,
                         ids=[f"B{b}H{h}q{nq}k{nk}D{d}{'c' if c else 'n'}s{s:g}" for b, h, nq, nk, d, c, s in SHAPES])
def test_shapes(B, H, Nq, Nk, D, causal, sigma):
    seed = 13 * Nk + Nq + D + causal
    q = rand((B, H, Nq, D), seed, sigma)
    k = rand((B, H, Nk, D), seed + 1, sigma)
    v = rand((B, H, Nk, D), seed + 2)
    scale = 1.0 / math.sqrt(D)
    o, lse = run(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention_decode(f64(q), f64(k), f64(v), causal, scale)
    check(o, lse, o_ref, lse_ref, f"B{B} H{H} Nq{Nq} Nk{Nk} D{D} causal={causal} sigma={sigma}")


def test_square_matches_the_forward_kernel():
    """Nq == Nk (<= 32) is the forward's problem: both kernels agree within rounding."""
    q, k, v = (t.cuda() for t in make_qkv(2, 2, 32, 128, seed=77))
    for causal in (False, True):
        o1, l1 = attn_decode(q, k, v, causal=causal)
        o2, l2 = attn_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
        assert (l1 - l2).abs().max().item() <= 1e-4


def test_rejects_unsupported():
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 1, 33, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="Nq"):
        attn_decode(q, k, k)
    with pytest.raises(ValueError):
        attn_decode(q[:, :, :8], k[:, :, :4], k[:, :, :4], causal=True)  # Nq > Nk
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="workspace"):
        attn_decode(q[:, :, :1], k, k, workspace=ws)


def test_workspace_reuse_is_bit_identical():
    dev = torch.device("cuda:0")
    q = rand((2, 2, 4, 64), 5).cuda()
    k, v = rand((2, 2, 700, 64), 6).cuda(), rand((2, 2, 700, 64), 7).cuda()
    ws = torch.full((decode_workspace_bytes(2, 2, 4, 700, 64),), 255, dtype=torch.uint8, device=dev)
    a = attn_decode(q, k, v, causal=True, workspace=ws)
    b = attn_decode(q, k, v, causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("wid", sorted(DECODE_WORKLOADS))
def test_decode_workloads_full(wid):
    w = DECODE_WORKLOADS[wid]
    print(f"[parity-decode] generating {w.describe()}", flush=True)
    q, k, v = decode_inputs(w)
    o, lse = run(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention_decode(f64(q), f64(k), f64(v), w.causal, w.scale)
    check(o, lse, o_ref, lse_ref, w.describe())
