"""GPU parity of the attention backward (dQ, dK, dV through the C ABI) against the fp64
backward oracle.

Inputs: seeded bf16 Q, K, V, dO; O and lse come from the library's forward on the GPU
(the backward's documented inputs), the oracle recomputes everything from Q, K, V, dO in
fp64. Bar per gradient tensor G (derived from the arithmetic: bf16 P and dS in the
matrix products, fp32 accumulation, Delta from the bf16 forward output, bf16 results):
  ||G_gpu - G_ref||_F / ||G_ref||_F <= 1e-2   and   max |G_gpu - G_ref| <= 2e-2 * max |G_ref|
and, where the reference gradient is zero (N = 1), max |G_gpu| <= 1e-4.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_fwd_amd import attn_bwd, attn_fwd, bwd_workspace_bytes
from softmax_attention_fwd_amd.inputs import WORKLOADS, make_dout, make_qkv, workload_inputs

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2
ZERO_ABS = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_grads(q, k, v, do, causal, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(name, got, ref, what):
    g = f64(got).reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite {name}"
    d = g - ref
    mx = float(np.abs(d).max())
    if np.linalg.norm(ref) < 1e-6:
        # the gradient vanishes (one key, or a row that only sees itself): only fp32
        # rounding of dP - Delta is left
        print(f"[parity-bwd] {what} {name}: reference is zero, max-abs {mx:.3e}", flush=True)
        assert mx <= ZERO_ABS, f"{what} {name}: max-abs {mx} where the gradient is zero"
        return
    rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
    bound = MAX_REL * float(np.abs(ref).max())
    print(f"[parity-bwd] {what} {name}: rel-L2 {rel:.3e} max-abs {mx:.3e} (bound {bound:.3e})",
          flush=True)
    assert rel <= REL_L2, f"{what} {name}: rel-L2 {rel}"
    assert mx <= bound, f"{what} {name}: max-abs {mx} > {bound}"


SMALL = [
    # B, H, N, D, causal, sigma_qk
    (1, 1, 1, 64, False, 1.0), (1, 1, 1, 128, True, 1.0),
    (1, 2, 17, 64, False, 1.0), (1, 2, 17, 64, True, 1.0),
    (2, 1, 100, 128, False, 1.0), (2, 1, 100, 128, True, 1.0),
    (1, 1, 129, 128, True, 1.0), (1, 3, 255, 64, True, 1.0),
    (2, 2, 257, 128, False, 1.0), (1, 2, 384, 64, False, 1.0),
    (2, 2, 384, 128, True, 1.0), (1, 1, 1000, 128, True, 1.0),
    (1, 2, 1536, 64, True, 2.0), (1, 2, 2048, 128, True, 2.0),
    (1, 1, 2048, 128, False, 1.0),
]


@pytest.mark.parametrize("B,H,N,D,causal,sigma", SMALL,
                         ids=[f"B{b}H{h}N{n}D{d}{'c' if c else 'n'}s{s:g}" for b, h, n, d, c, s in SMALL])
def test_small_shapes(B, H, N, D, causal, sigma):
    q, k, v = make_qkv(B, H, N, D, seed=11 * N + D + causal, sigma_q=sigma, sigma_k=sigma)
    do = make_dout(B, H, N, D, seed=11 * N + D + causal)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = gpu_grads(q, k, v, do, causal, scale)
    rq, rk, rv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), causal, scale)
    what = f"B{B} H{H} N{N} D{D} causal={causal} sigma={sigma}"
    check("dQ", dq, rq, what)
    check("dK", dk, rk, what)
    check("dV", dv, rv, what)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_value_rows_give_small_dq_dk(causal):
    """Equal V rows make dS vanish (dP_ij is the same for every j and equals Delta_i), so
    dQ and dK are zero up to the rounding of the forward output that Delta is formed from."""
    q, k, v = make_qkv(1, 2, 200, 128, seed=71)
    v = v[:, :, :1, :].expand(-1, -1, 200, -1).contiguous()
    do = make_dout(1, 2, 200, 128, seed=71)
    dq, dk, dv = gpu_grads(q, k, v, do, causal, 1 / math.sqrt(128))
    _, _, rv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), causal, 1 / math.sqrt(128))
    scale_ref = float(np.abs(f64(dv)).max())
    assert float(dq.abs().max()) <= 2e-2 * scale_ref and float(dk.abs().max()) <= 2e-2 * scale_ref
    check("dV", dv, rv, f"equal V rows causal={causal}")


def test_workspace_and_outputs_in_place():
    """Given outputs and a workspace are written in place; a second call with a dirty
    workspace gives bit-identical results."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_qkv(2, 2, 300, 64, seed=73))
    do = make_dout(2, 2, 300, 64, seed=73).to(dev)
    o, lse = attn_fwd(q, k, v, causal=True)
    ws = torch.full((bwd_workspace_bytes(2, 2, 300),), 255, dtype=torch.uint8, device=dev)
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    r1 = attn_bwd(q, k, v, o, do, lse, causal=True, dq=outs[0], dk=outs[1], dv=outs[2], workspace=ws)
    assert all(a is b for a, b in zip(r1, outs))
    first = [t.clone() for t in r1]
    r2 = attn_bwd(q, k, v, o, do, lse, causal=True, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(first, r2):
        assert torch.isfinite(a).all() and torch.equal(a, b)


def test_rejects_small_workspace():
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_qkv(1, 1, 64, 64, seed=1))
    o, lse = attn_fwd(q, k, v)
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="workspace"):
        attn_bwd(q, k, v, o, q, lse, workspace=ws)


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_workload_full_size(wid):
    """The workloads' shapes at full size, every element against the oracle (run on the
    host cores, 16 heads at a time)."""
    from threadpoolctl import threadpool_limits

    w = WORKLOADS[wid]
    print(f"[parity-bwd] generating {w.describe()}", flush=True)
    q, k, v = workload_inputs(w)
    do = make_dout(w.B, w.H, w.N, w.D, seed=w.seed)
    dq, dk, dv = (t.cpu() for t in gpu_grads(q, k, v, do, w.causal, w.scale))
    workers = min(16, len(os.sched_getaffinity(0)))
    nh = w.B * w.H
    flat = [t.view(nh, 1, w.N, w.D) for t in (q, k, v, do)]
    got = [t.view(nh, w.N, w.D) for t in (dq, dk, dv)]
    stats = {n: [0.0, 0.0, 0.0, 0.0] for n in ("dQ", "dK", "dV")}  # diff2, ref2, maxdiff, maxref
    with threadpool_limits(limits=1):
        for h0 in range(0, nh, 16):
            h1 = min(nh, h0 + 16)
            refs = oracle.attention_bwd(*(f64(t[h0:h1]).swapaxes(0, 1) for t in flat), w.causal,
                                        w.scale, workers=workers)
            for name, g, r in zip(("dQ", "dK", "dV"), got, refs):
                d = f64(g[h0:h1]) - r[0]
                assert np.isfinite(d).all(), f"non-finite {name}"
                st = stats[name]
                st[0] += float((d * d).sum())
                st[1] += float((r * r).sum())
                st[2] = max(st[2], float(np.abs(d).max()))
                st[3] = max(st[3], float(np.abs(r).max()))
    for name, (d2, r2, md, mr) in stats.items():
        rel = math.sqrt(d2 / r2)
        print(f"[parity-bwd] {w.describe()} {name}: rel-L2 {rel:.3e} max-abs {md:.3e} "
              f"(bound {MAX_REL * mr:.3e})", flush=True)
        assert rel <= REL_L2 and md <= MAX_REL * mr, name
