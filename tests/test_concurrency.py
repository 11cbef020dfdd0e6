"""Concurrent use of the library from one process (GPU tests).

Every entry point is called from two host threads at once. Each thread works on its own
stream, with its own inputs, outputs and workspaces, and must get bit for bit what serial
calls on the default stream return. The kernels use no atomics and fixed reduction orders,
so any difference would come from state shared between calls. The threads run before the
serial reference: in a fresh process they also touch the host-side caches (compute-unit
counts) for the first time together, which exercises their locking.
"""
from __future__ import annotations

import threading

import pytest
import torch

from softmax_attention_fwd_amd import attn_bwd, attn_decode, attn_fwd, based_fwd, gemm_nt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def randn(g, *shape):
    return torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()


def job(seed: int):
    """One round of every operation on small, ragged shapes; returns the outputs."""
    g = torch.Generator().manual_seed(seed)
    causal = bool(seed % 2)
    B, H, N, D = 2, 3, 600 + 37 * seed, 128
    q, k, v, do = (randn(g, B, H, N, D) for _ in range(4))
    o, lse = attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = attn_bwd(q, k, v, o, do, lse, causal=causal)
    qd = q[:, :, : 3 + seed].contiguous()
    od, ld = attn_decode(qd, k, v, causal=True)
    a, b = randn(g, 300 + seed, 256), randn(g, 264, 256)
    c = gemm_nt(a, b)
    bq, bk, bv = randn(g, 1, 2, 2000 + seed, 16), randn(g, 1, 2, 2000 + seed, 16), randn(g, 1, 2, 2000 + seed, 64)
    ob = based_fwd(bq, bk, bv)  # 2 heads: the split launch with a workspace
    # the persistent forward grids: 512 (long, short) causal query-tile pairs, or 512 units
    Hp = 32 if causal else 16
    qp, kp, vp = (randn(g, 4, Hp, 2048, 128) for _ in range(3))
    op, lp = attn_fwd(qp, kp, vp, causal=causal)
    return [o, lse, dq, dk, dv, od, ld, c, ob, op, lp]


def test_two_threads_on_two_streams_match_serial():
    seeds = (1, 2)
    results, errors = {}, []

    def worker(seed):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                out = None
                for _ in range(3):
                    out = job(seed)
                stream.synchronize()
            results[seed] = out
        except Exception as exc:  # reported below, in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(s,)) for s in seeds]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=300)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, f"worker raised: {errors[0]!r}"
    serial = {s: job(s) for s in seeds}
    torch.cuda.synchronize()
    names = ["o", "lse", "dq", "dk", "dv", "decode o", "decode lse", "gemm c", "based o",
             "persistent o", "persistent lse"]
    for s in seeds:
        for name, x, y in zip(names, serial[s], results[s]):
            assert torch.equal(x, y), f"seed {s}: {name} differs from the serial result"
