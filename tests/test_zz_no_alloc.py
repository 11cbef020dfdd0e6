"""GPU check of attn_decode_noalloc, the decode entry point that allocates nothing (its
per-chunk partials live in a fixed device array inside the library), through the C ABI:
on consecutive calls, the second on a smaller problem than the first, its output must
equal attn_decode's (the same kernels on a caller workspace) bit for bit, and both are
held to the fp64 decode oracle with the forward's bar (O max-abs <= 2e-2, rel-L2 <= 5e-3,
lse max-abs <= 1e-3). A problem larger than the fixed array is rejected.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_fwd_amd import attn_decode, attn_decode_noalloc, decode_workspace_bytes
from softmax_attention_fwd_amd.inputs import DECODE_WORKLOADS, decode_inputs, make_qkv

pytestmark = pytest.mark.gpu

NOALLOC_MAX = 33 << 20  # ATTN_DECODE_NOALLOC_MAX_WORKSPACE


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def bar(o, lse, o_ref, lse_ref, what):
    og, lg = f64(o), f64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), f"{what}: non-finite output"
    d = og - o_ref
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / np.linalg.norm(o_ref))
    lse_err = float(np.abs(lg - lse_ref).max())
    print(f"[no-alloc] {what}: O max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse max-abs {lse_err:.3e}",
          flush=True)
    assert max_abs <= 2e-2 and rel <= 5e-3 and lse_err <= 1e-3, what


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    dev = torch.device("cuda:0")
    w = DECODE_WORKLOADS[2]  # B1 H32, 8 queries against 16384 peaky keys: 32 chunks per head
    big = decode_inputs(w) + (w.causal, w.scale)
    q, k, v = make_qkv(1, 3, 700, 64, seed=5)
    small = (q[:, :, -3:, :].contiguous(), k, v, False, 0.125)  # 3 queries, 700 keys, D 64
    cases = [("big", big), ("small", small)]
    for name, (q, k, v, causal, scale) in cases:
        need = decode_workspace_bytes(*q.shape[:3], k.shape[2], q.shape[3])
        assert 0 < need <= NOALLOC_MAX
    results = []
    for name, (q, k, v, causal, scale) in cases:  # the no-alloc calls back to back
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
        print(f"[no-alloc] call {name}: q {tuple(q.shape)} k {tuple(k.shape)} causal={causal}", flush=True)
        attn_decode_noalloc(qd, kd, vd, causal=causal, scale=scale, out=o, lse=lse)
        results.append((o, lse))
    torch.cuda.synchronize()
    for (name, (q, k, v, causal, scale)), (o, lse) in zip(cases, results):
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o_ws, lse_ws = attn_decode(qd, kd, vd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws), f"{name}: O differs from attn_decode"
        assert torch.equal(lse, lse_ws), f"{name}: lse differs from attn_decode"
        o_ref, lse_ref = oracle.attention_decode(f64(q), f64(k), f64(v), causal, scale)
        bar(o, lse, o_ref, lse_ref, name)


def test_noalloc_repeat_after_smaller_call():
    # the fixed array keeps the last call's partials: a call after a smaller one must not
    # read any of them
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(4, 8, 4096, 128, seed=9)
    qd, kd, vd = q[:, :, -2:, :].contiguous().to(dev), k.to(dev), v.to(dev)
    o1, l1 = attn_decode_noalloc(qd, kd, vd, causal=True)
    o2, l2 = attn_decode_noalloc(qd[:1, :2].contiguous(), kd[:1, :2, :1000].contiguous(),
                                 vd[:1, :2, :1000].contiguous(), causal=True)
    o3, l3 = attn_decode_noalloc(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    o_ws, l_ws = attn_decode(qd[:1, :2].contiguous(), kd[:1, :2, :1000].contiguous(),
                             vd[:1, :2, :1000].contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ws) and torch.equal(l2, l_ws)


def test_noalloc_rejects_problem_beyond_scratch():
    dev = torch.device("cuda:0")
    B, H, Nq, Nk, D = 64, 64, 32, 256, 128  # B*H = 4096 heads of 32 queries: 64 MiB of partials
    assert decode_workspace_bytes(B, H, Nq, Nk, D) > NOALLOC_MAX
    q = torch.zeros((B, H, Nq, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, H, Nk, D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="code -5"):
        attn_decode_noalloc(q, k, k, causal=False)
