"""Seeded synthetic inputs and the five attention workloads.

This module draws random numbers and nothing else: it holds none of the attention
arithmetic, so both the HIP path's tests and the CPU oracle can take their inputs from
it without sharing any of the method.

Recipe (the pages fix none; the same recipe serves tests and the benchmark):
  one CPU ``torch.Generator`` per call, seeded with ``seed``; draw Q, then K, then V as
  float32 standard normals of shape [B, H, N, D]; multiply each by its sigma; round to
  bfloat16 with round-to-nearest-even (torch's float32 -> bfloat16 cast).
The workloads use seed 1000 + workload number. The backward's incoming gradient dO is
drawn the same way from its own generator (``make_dout``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, mask, input scales."""
    name: str
    B: int
    H: int
    N: int
    D: int
    causal: bool
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """4*B*H*N^2*D, halved when causal (the throughput convention of the metric)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.D
        return f / 2 if self.causal else f

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once and O written once (bf16), lse (fp32)."""
        return 4 * self.B * self.H * self.N * self.D * 2 + self.B * self.H * self.N * 4

    def describe(self) -> str:
        c = "causal" if self.causal else "non-causal"
        return f"B{self.B} H{self.H} N{self.N} D{self.D} {c}"


# The five workloads: small parity case, two non-causal, two causal (the last with
# Q, K ~ N(0, 2^2) so the softmax is peaky and the rescaling is exercised hard).
WORKLOADS = {
    1: Workload("w1_b1h1n128d64", 1, 1, 128, 64, False, seed=1001),
    2: Workload("w2_b16h16n1024d64", 16, 16, 1024, 64, False, seed=1002),
    3: Workload("w3_b16h16n4096d128", 16, 16, 4096, 128, False, seed=1003),
    4: Workload("w4_b8h32n8192d128_causal", 8, 32, 8192, 128, True, seed=1004),
    5: Workload("w5_b1h32n16384d128_causal_sigma2", 1, 32, 16384, 128, True,
                sigma_q=2.0, sigma_k=2.0, seed=1005),
}


def make_qkv(B: int, H: int, N: int, D: int, seed: int, sigma_q: float = 1.0,
             sigma_k: float = 1.0, sigma_v: float = 1.0):
    """Q, K, V as contiguous CPU bfloat16 tensors of shape [B, H, N, D]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for sigma in (sigma_q, sigma_k, sigma_v):
        x = torch.randn((B, H, N, D), generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out.append(x.to(torch.bfloat16).contiguous())
    return tuple(out)


def workload_inputs(w: Workload):
    """Q, K, V (CPU bfloat16) of a workload, from its own seed."""
    return make_qkv(w.B, w.H, w.N, w.D, w.seed, w.sigma_q, w.sigma_k, w.sigma_v)


def make_dout(B: int, H: int, N: int, D: int, seed: int, sigma: float = 1.0):
    """An incoming gradient dO for the backward pass: CPU bfloat16 [B, H, N, D] standard
    normals times sigma, from a generator seeded with ``seed`` + 7919 (so it differs from
    the Q, K, V of the same seed)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    x = torch.randn((B, H, N, D), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16).contiguous()


@dataclass(frozen=True)
class DecodeWorkload:
    """A decode-shaped problem: Nq queries against an Nk-long key/value sequence."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    causal: bool
    sigma_qk: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def kv_bytes(self) -> int:
        """K and V read once (bf16): the bytes that bound the kernel."""
        return 2 * self.B * self.H * self.Nk * self.D * 2

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: K, V, Q read once, O (bf16) and lse (fp32) written."""
        return self.kv_bytes + 2 * self.B * self.H * self.Nq * self.D * 2 + 4 * self.B * self.H * self.Nq

    def describe(self) -> str:
        c = "causal" if self.causal else "non-causal"
        return f"B{self.B} H{self.H} Nq{self.Nq} Nk{self.Nk} D{self.D} {c}"


# Decode shapes built from the forward workloads' heads and lengths (the pages give no
# inference shapes): one new token per sequence against the KV cache of workload 3's
# batch, 8 speculative tokens against workload 5's long peaky sequence, and one token
# against a 128K-token cache.
DECODE_WORKLOADS = {
    1: DecodeWorkload("d1_b16h16q1k4096d128", 16, 16, 1, 4096, 128, True, seed=2001),
    2: DecodeWorkload("d2_b1h32q8k16384d128", 1, 32, 8, 16384, 128, True, sigma_qk=2.0, seed=2002),
    3: DecodeWorkload("d3_b4h8q1k131072d128", 4, 8, 1, 131072, 128, True, seed=2003),
}


def decode_inputs(w: DecodeWorkload):
    """Q [B, H, Nq, D], K, V [B, H, Nk, D] (CPU bfloat16) of a decode workload: one
    generator seeded with w.seed draws Q, then K, then V (standard normals; Q and K times
    sigma_qk), rounded to bfloat16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    out = []
    for shape, sigma in (((w.B, w.H, w.Nq, w.D), w.sigma_qk), ((w.B, w.H, w.Nk, w.D), w.sigma_qk),
                         ((w.B, w.H, w.Nk, w.D), 1.0)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out.append(x.to(torch.bfloat16).contiguous())
    return tuple(out)


@dataclass(frozen=True)
class BasedWorkload:
    """A Based linear-attention problem: q, k [B, H, N, d], v [B, H, N, dv], causal."""
    name: str
    B: int
    H: int
    N: int
    d: int = 16
    dv: int = 64
    seed: int = 0

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: q, k, v read once and o written once, all bf16."""
        return 2 * self.B * self.H * self.N * (2 * self.d + 2 * self.dv)

    @property
    def flops(self) -> int:
        """Algorithmic flop of the chunked linear-time form with 64-token chunks: per token
        2 * 273 * dv for the state update and 2 * 273 * dv for the inter-chunk product, and
        per chunk pair (query, key) inside the chunk (64 * 65 / 2 of them) 2 * (d + dv)."""
        F = 1 + self.d + self.d * self.d
        n_chunks = -(-self.N // 64)
        intra = n_chunks * (64 * 65 // 2) * 2 * (self.d + self.dv)
        return self.B * self.H * (4 * F * self.dv * self.N + intra)

    def describe(self) -> str:
        return f"B{self.B} H{self.H} N{self.N} d{self.d} dv{self.dv} causal"


# Based shapes: the published design's 16 query/key features and 64-wide heads, on the
# batch, heads and length of the attention forward's workload 3, and a longer sequence.
BASED_WORKLOADS = {
    1: BasedWorkload("b1_b2h4n1024", 2, 4, 1024, seed=3001),
    2: BasedWorkload("b2_b16h16n4096", 16, 16, 4096, seed=3002),
    3: BasedWorkload("b3_b4h16n16384", 4, 16, 16384, seed=3003),
}


def based_inputs(w: BasedWorkload):
    """q, k [B, H, N, d] and v [B, H, N, dv] (CPU bfloat16): one generator seeded with
    w.seed draws q, then k, then v as standard normals, rounded to bfloat16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    out = []
    for dim in (w.d, w.d, w.dv):
        out.append(torch.randn((w.B, w.H, w.N, dim), generator=g, dtype=torch.float32)
                   .to(torch.bfloat16).contiguous())
    return tuple(out)
