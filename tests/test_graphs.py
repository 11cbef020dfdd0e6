"""Graph capture of the library's entry points (GPU tests).

Serving loops capture a sequence of calls into a HIP graph once and replay it. The entry
points only enqueue kernels on the stream they are handed: they allocate no device memory,
record no memset and never synchronise. So a captured sequence must replay to exactly the
bits that eager calls give on the same inputs, and must follow new values written into the
captured input buffers. Each replay is checked, with eager work and synchronisations between
replays. The shapes take the persistent grids of the forward (non-causal D = 128 and D = 64,
and the causal grid of long/short query-tile pairs) as well as a one-unit-per-workgroup
launch, the decode entry point that uses the library's own scratch array, the backward with
its workspace, the GEMM and Based.
"""
from __future__ import annotations

import pytest
import torch

from softmax_attention_fwd_amd import (attn_bwd, attn_decode_noalloc, attn_fwd, based_fwd,
                                       gemm_nt)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


# name -> shapes of its bf16 inputs
SHAPES = {
    "fwd_d128": [(4, 16, 2048, 128)] * 3,             # 512 units: persistent grid
    "fwd_d128_causal": [(4, 32, 2048, 128)] * 3,      # 512 (long, short) pairs: persistent
    "fwd_d64": [(8, 16, 2048, 64)] * 3,               # 512 units of 512 queries: persistent
    "fwd_small": [(1, 2, 300, 64)] * 3,               # one unit per workgroup, ragged
    "decode": [(4, 8, 4, 128), (4, 8, 8192, 128), (4, 8, 8192, 128)],
    "bwd": [(1, 4, 1000, 128)] * 4,                   # q, k, v, dO
    "gemm": [(1000, 256), (520, 256)],
    "based": [(1, 2, 2000, 16), (1, 2, 2000, 16), (1, 2, 2000, 64)],
}


def fill(tensors, seed):
    """Write fresh seeded N(0, 1) values into the given buffers, in place."""
    g = torch.Generator().manual_seed(seed)
    for t in tensors:
        t.copy_(torch.randn(*t.shape, generator=g).to(torch.bfloat16))


def run(x):
    """Every captured call, on the static inputs x; returns the outputs in a fixed order."""
    outs = []
    outs += attn_fwd(*x["fwd_d128"])
    outs += attn_fwd(*x["fwd_d128_causal"], causal=True)
    outs += attn_fwd(*x["fwd_d64"])
    outs += attn_fwd(*x["fwd_small"], causal=True)
    outs += attn_decode_noalloc(*x["decode"], causal=True)
    q, k, v, do = x["bwd"]
    o, lse = attn_fwd(q, k, v, causal=True)
    outs += [o, lse, *attn_bwd(q, k, v, o, do, lse, causal=True)]
    outs.append(gemm_nt(*x["gemm"]))
    outs.append(based_fwd(*x["based"]))
    return outs


def test_captured_sequence_replays_to_eager_bits():
    x = {name: [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
         for name, shapes in SHAPES.items()}
    inputs = [t for ts in x.values() for t in ts]
    fill(inputs, 100)
    # warm up on a side stream: first calls fill the library's per-device caches
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static_out = run(x)
    torch.cuda.synchronize()

    for replay, seed in enumerate((101, 102, 101, 103)):
        fill(inputs, seed)
        graph.replay()
        torch.cuda.synchronize()
        captured = [t.clone() for t in static_out]
        eager = run(x)  # eager work between replays, on the same inputs
        torch.cuda.synchronize()
        assert len(captured) == len(eager)
        for i, (a, b) in enumerate(zip(captured, eager)):
            assert torch.isfinite(b.float()).all(), f"replay {replay}: eager output {i} not finite"
            assert torch.equal(a, b), f"replay {replay} (seed {seed}): output {i} differs from eager"
