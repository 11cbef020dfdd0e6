"""GPU parity of the bf16 GEMM (C = A B^T through the C ABI) against the fp64 oracle.

Bar (from the arithmetic: bf16 inputs are exact in fp32, the K products accumulate in
fp32, C is rounded once to bf16 to nearest even): per element
  |C - C_ref| <= 2^-8 |C_ref| + 2 K 2^-24 (|A| |B|^T)
i.e. the largest relative bf16 rounding (half an ulp at the bottom of a binade) plus the
classical bound on an fp32 sum of K products, doubled.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_fwd_amd import gemm_nt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


SHAPES = [(1, 8, 8), (7, 16, 24), (256, 256, 64), (255, 264, 72), (300, 512, 1000),
          (1024, 1024, 1024), (513, 8, 4096), (2048, 1536, 512), (4096, 4096, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES, ids=[f"M{m}N{n}K{k}" for m, n, k in SHAPES])
def test_gemm(M, N, K):
    a, b = rand((M, K), M + K), rand((N, K), N + 3 * K)
    c = gemm_nt(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    ref = oracle.gemm_nt(a.double().numpy(), b.double().numpy())
    got = c.double().cpu().numpy()
    absprod = oracle.gemm_nt(np.abs(a.double().numpy()), np.abs(b.double().numpy()))
    bound = 2.0 ** -8 * np.abs(ref) + 2 * K * 2.0 ** -24 * absprod
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"[parity-gemm] M{M} N{N} K{K}: max err/bound {float((err / bound).max()):.3f} rel-L2 {rel:.2e}",
          flush=True)
    assert np.isfinite(got).all()
    assert (err <= bound).all()


def test_gemm_writes_nothing_outside_c():
    M, N, K = 100, 40, 64
    a, b = rand((M, K), 1).cuda(), rand((N, K), 2).cuda()
    buf = torch.full((M * N + 512,), 7.0, dtype=torch.bfloat16, device="cuda")
    c = buf[256:256 + M * N].view(M, N)
    gemm_nt(a, b, out=c)
    torch.cuda.synchronize()
    assert (buf[:256] == 7.0).all() and (buf[256 + M * N:] == 7.0).all()
    ref = oracle.gemm_nt(a.double().cpu().numpy(), b.double().cpu().numpy())
    assert np.abs(c.double().cpu().numpy() - ref).max() <= 2.0 ** -8 * np.abs(ref).max() + 1e-3


def test_gemm_bench_shape_sampled_rows():
    """The launch the benchmark times (M = N = K = 8192): 16 rows of C (first, last, tile
    edges and random ones) against the oracle, per element, and the whole C finite."""
    M = N = K = 8192
    a, b = rand((M, K), 8192), rand((N, K), 8193)
    c = gemm_nt(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(c.float()).all()
    rng = np.random.default_rng(5)
    rows = sorted({0, 1, 255, 256, 4095, 4096, 8191} | set(int(r) for r in rng.integers(0, M, 9)))
    an, bn = a[rows].double().numpy(), b.double().numpy()
    ref = oracle.gemm_nt(an, bn)
    absprod = oracle.gemm_nt(np.abs(an), np.abs(bn))
    bound = 2.0 ** -8 * np.abs(ref) + 2 * K * 2.0 ** -24 * absprod
    got = c[rows].double().cpu().numpy()
    err = np.abs(got - ref)
    print(f"[parity-gemm] 8192^3 rows {rows}: max err/bound {float((err / bound).max()):.3f}", flush=True)
    assert (err <= bound).all()
