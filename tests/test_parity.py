"""GPU parity: the HIP attention forward, called through the C ABI, against the fp64 oracle.

Bar (derived from the arithmetic: bf16 inputs, fp32 scores and softmax state, bf16 P for
the P*V product, bf16 output rounded to nearest even):
  O:   max |O_gpu - O_ref| <= 2e-2 and ||O_gpu - O_ref||_F / ||O_ref||_F <= 5e-3
  lse: max |lse_gpu - lse_ref| <= 1e-3
Small shapes compare every element with the full oracle; the five workloads at their full
sizes (the launch the benchmark times) compare sampled rows with the per-row oracle and
check whole-tensor properties that hold at any size.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_fwd_amd import attn_fwd
from softmax_attention_fwd_amd.inputs import WORKLOADS, make_qkv, workload_inputs

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    return torch.device("cuda:0")


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def run(q, k, v, causal, scale=None, **kw):
    dev = torch.device("cuda:0")
    o, lse = attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def check(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    og = f64(o_gpu).reshape(o_ref.shape)
    lg = f64(lse_gpu).reshape(lse_ref.shape)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), f"non-finite output {what}"
    d = og - o_ref
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(o_ref), 1e-300))
    lse_err = float(np.abs(lg - lse_ref).max())
    print(f"[parity] {what}: O max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse max-abs {lse_err:.3e}",
          flush=True)
    assert max_abs <= O_MAX_ABS, f"{what}: O max-abs {max_abs}"
    assert rel <= O_REL_L2, f"{what}: O rel-L2 {rel}"
    assert lse_err <= LSE_MAX_ABS, f"{what}: lse max-abs {lse_err}"
    return max_abs, rel, lse_err


# ---------------------------------------------------------------- small shapes, full oracle

SMALL = [
    # B, H, N, D, causal, sigma_qk
    (1, 1, 1, 64, False, 1.0), (1, 1, 1, 128, True, 1.0),
    (1, 2, 17, 64, False, 1.0), (1, 2, 17, 64, True, 1.0),
    (2, 1, 100, 128, False, 1.0), (2, 1, 100, 128, True, 1.0),
    (1, 1, 129, 128, False, 1.0), (1, 1, 129, 64, True, 1.0),
    (1, 3, 255, 64, True, 1.0), (2, 2, 257, 128, False, 1.0),
    (1, 2, 384, 64, False, 1.0), (2, 4, 384, 128, True, 1.0),   # grid multiple of 8
    (1, 1, 1000, 128, True, 1.0), (1, 1, 1000, 64, False, 1.0),
    (1, 2, 2048, 128, True, 2.0), (1, 2, 1536, 64, False, 2.0),
    (1, 1, 4096, 128, False, 1.0), (1, 1, 4095, 128, True, 1.0),
]


@pytest.mark.parametrize("B,H,N,D,causal,sigma", SMALL,
                         ids=[f"B{b}H{h}N{n}D{d}{'c' if c else 'n'}s{s:g}" for b, h, n, d, c, s in SMALL])
def test_small_shapes_full_oracle(B, H, N, D, causal, sigma):
    seed = 7 * N + D + (1 if causal else 0)
    q, k, v = make_qkv(B, H, N, D, seed=seed, sigma_q=sigma, sigma_k=sigma)
    scale = 1.0 / math.sqrt(D)
    o, lse = run(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), causal, scale)
    check(o, lse, o_ref, lse_ref, f"B{B} H{H} N{N} D{D} causal={causal} sigma={sigma}")


# Both forward kernels (ping-pong, the D = 128 default and the non-causal D = 64 default on
# grids that fill the device, and four-wave, the other D = 64 default) can be forced per
# call through attn_fwd_ex. They perform the same per-row arithmetic in the same order,
# so their outputs must agree bit for bit; each is also held to the oracle on the
# non-default head dimension. The shapes include grids of more workgroups than the GPU
# holds at once.
KERNEL_PAIRS = [
    # B, H, N, D, causal
    (1, 1, 1, 64, False), (1, 2, 17, 128, True), (2, 1, 300, 64, True),
    (2, 2, 257, 64, False), (1, 2, 1000, 128, False), (2, 4, 384, 128, True),
    (1, 1, 4095, 128, True), (3, 5, 1024, 64, True), (4, 8, 4096, 128, False),
    (2, 8, 8192, 128, True), (1, 1, 256, 128, False), (16, 20, 256, 128, False),
    (8, 16, 768, 128, False), (64, 16, 512, 128, False),
]


@pytest.mark.parametrize("B,H,N,D,causal", KERNEL_PAIRS,
                         ids=[f"B{b}H{h}N{n}D{d}{'c' if c else 'n'}" for b, h, n, d, c in KERNEL_PAIRS])
def test_kernels_bit_identical(B, H, N, D, causal):
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, D, seed=11 * N + D))
    out = {kernel: run(q, k, v, causal, kernel=kernel) for kernel in ("pingpong", "fourwave")}
    default = run(q, k, v, causal)
    (o_p, l_p), (o_f, l_f) = out["pingpong"], out["fourwave"]
    assert torch.equal(o_p, o_f), f"O differs: max {(o_p.float() - o_f.float()).abs().max().item()}"
    assert torch.equal(l_p, l_f), f"lse differs: max {(l_p - l_f).abs().max().item()}"
    assert torch.equal(default[0], o_p) and torch.equal(default[1], l_p)


# Non-causal grids of more work units than compute units, ragged N (last key tile and last
# query tile partial, down to one row), unit counts that are and are not multiples of 8
# (XCD order on and off) and both head sizes: the ping-pong and four-wave kernels must agree
# bit for bit, and sampled rows of the first and last head match the oracle. At D = 128 a
# workgroup loads its next unit's first tiles and Q rows during the current unit's last
# pair, also after a unit whose last waves are idle (N = 4097, 300).
LARGE_GRID_SHAPES = [
    # B, H, N, D
    (16, 20, 256, 128), (64, 16, 512, 128), (16, 16, 1024, 64), (5, 9, 2500, 64),
    (11, 7, 1000, 128), (4, 5, 4097, 128), (2, 130, 300, 128),
    # a workgroup's next unit has a ragged K(0) (N < 64) or K(1) (64 < N < 128)
    (4, 80, 50, 128), (3, 100, 100, 128),
    # persistent D = 64 grids (more than 256 units of 512 queries) with ragged units: idle
    # waves and partly filled query blocks
    (4, 80, 50, 64), (3, 100, 545, 64), (2, 100, 1600, 64),
    # D = 64 ping-pong waves hold two 32-query blocks: a last wave whose second block is
    # partly past N (545 = 512 + 33) and one whose second block is wholly past it (1600)
    (3, 5, 545, 64), (7, 3, 1600, 64),
]


@pytest.mark.parametrize("B,H,N,D", LARGE_GRID_SHAPES, ids=[f"B{b}H{h}N{n}D{d}" for b, h, n, d in LARGE_GRID_SHAPES])
def test_large_grids_bit_identical(B, H, N, D):
    print(f"[large grid] B{B} H{H} N{N} D{D}", flush=True)
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, D, seed=19 * N + D + B))
    o_p, l_p = run(q, k, v, False, kernel="pingpong")
    o_f, l_f = run(q, k, v, False, kernel="fourwave")
    assert torch.equal(o_p, o_f), f"O differs: max {(o_p.float() - o_f.float()).abs().max().item()}"
    assert torch.equal(l_p, l_f), f"lse differs: max {(l_p - l_f).abs().max().item()}"
    rows = np.random.default_rng(N).choice(N, size=min(N, 96), replace=False)
    rows.sort()
    qd, kd, vd = f64(q.cpu()), f64(k.cpu()), f64(v.cpu())
    for bh in (0, B * H - 1):
        b, h = divmod(bh, H)
        o_ref, lse_ref = oracle.attention_rows(qd, kd, vd, [(b, h, int(i)) for i in rows], False,
                                               1 / math.sqrt(D))
        check(o_p[b, h][rows], l_p[b, h][rows], o_ref, lse_ref, f"large grid B{B} H{H} N{N} D{D} head {bh}")


# Causal D = 128 grids with more units than compute units. When a head's query tiles pair up
# and the pairs split evenly over the grid, a persistent grid walks (long, short) pairs and
# loads each next unit's first tiles and Q rows early; B4 H32 N900 (ragged, idle waves in
# the last tile) and B8 H32 N2048 do, B2 H64 N1536 (384 pairs) falls back to one unit per
# workgroup. The ping-pong and four-wave kernels agree bit for bit; sampled rows of the first
# and last head match the oracle.
CAUSAL_GRID_SHAPES = [(4, 32, 900, 128), (8, 32, 2048, 128), (2, 64, 1536, 128)]


@pytest.mark.parametrize("B,H,N,D", CAUSAL_GRID_SHAPES, ids=[f"B{b}H{h}N{n}D{d}" for b, h, n, d in CAUSAL_GRID_SHAPES])
def test_causal_grids_bit_identical(B, H, N, D):
    print(f"[causal grid] B{B} H{H} N{N} D{D}", flush=True)
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, D, seed=23 * N + D + B))
    o_p, l_p = run(q, k, v, True, kernel="pingpong")
    o_f, l_f = run(q, k, v, True, kernel="fourwave")
    assert torch.equal(o_p, o_f), f"O differs: max {(o_p.float() - o_f.float()).abs().max().item()}"
    assert torch.equal(l_p, l_f), f"lse differs: max {(l_p - l_f).abs().max().item()}"
    default = run(q, k, v, True)
    assert torch.equal(default[0], o_p) and torch.equal(default[1], l_p)
    rows = np.random.default_rng(N + 1).choice(N, size=min(N, 96), replace=False)
    rows.sort()
    qd, kd, vd = f64(q.cpu()), f64(k.cpu()), f64(v.cpu())
    for bh in (0, B * H - 1):
        b, h = divmod(bh, H)
        o_ref, lse_ref = oracle.attention_rows(qd, kd, vd, [(b, h, int(i)) for i in rows], True,
                                               1 / math.sqrt(D))
        check(o_p[b, h][rows], l_p[b, h][rows], o_ref, lse_ref, f"causal grid B{B} H{H} N{N} D{D} head {bh}")


# More workgroups than the GPU holds at once (640 and 512 at D = 128, one per compute unit
# at a time): every element against the oracle, so that a workgroup that reads or stores
# another unit's rows cannot pass.
@pytest.mark.parametrize("B,H,N", [(16, 40, 256), (8, 16, 1024)])
def test_many_workgroups_full_oracle(B, H, N):
    q, k, v = make_qkv(B, H, N, 128, seed=17 * N + H)
    o, lse = run(q, k, v, False)
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), False, 1 / math.sqrt(128))
    check(o, lse, o_ref, lse_ref, f"B{B} H{H} N{N} D128")


@pytest.mark.parametrize("kernel,D", [("pingpong", 64), ("fourwave", 128)])
@pytest.mark.parametrize("N,causal", [(1, False), (129, True), (1000, False), (2048, True)])
def test_non_default_kernel_full_oracle(kernel, D, N, causal):
    q, k, v = make_qkv(2, 3, N, D, seed=13 * N + D)
    o, lse = run(q, k, v, causal, kernel=kernel)
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), causal, 1 / math.sqrt(D))
    check(o, lse, o_ref, lse_ref, f"{kernel} N{N} D{D} causal={causal}")


def test_workload1_full_oracle():
    w = WORKLOADS[1]
    q, k, v = workload_inputs(w)
    o, lse = run(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), w.causal, w.scale)
    check(o, lse, o_ref, lse_ref, w.describe())


@pytest.mark.parametrize("scale", [0.01, 0.5, 2.0])
def test_other_scales(scale):
    q, k, v = make_qkv(1, 2, 300, 64, seed=31)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, scale)
        o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), causal, scale)
        check(o, lse, o_ref, lse_ref, f"scale={scale} causal={causal}")


# ---------------------------------------------------------------- closed forms through the GPU

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_value_rows(D, causal):
    q, k, v = make_qkv(2, 2, 333, D, seed=41, sigma_q=2.0, sigma_k=2.0)
    v = v[:, :, :1, :].expand(-1, -1, 333, -1).contiguous()
    o, _ = run(q, k, v, causal)
    err = (o.float().cpu() - v.float()).abs().max().item()
    # only the bf16 rounding of P (relative 2^-9) and of O separate O from v
    assert err <= 4 * 2.0 ** -8 * v.float().abs().max().item() + 1e-6, err


@pytest.mark.parametrize("D", [64, 128])
def test_causal_row0_exact(D):
    q, k, v = make_qkv(3, 2, 200, D, seed=43, sigma_q=2.0, sigma_k=2.0)
    scale = 1.0 / math.sqrt(D)
    o, lse = run(q, k, v, True, scale)
    assert torch.equal(o[:, :, 0, :].cpu(), v[:, :, 0, :]), "row 0 must equal V[0] exactly"
    want = scale * (q[:, :, 0, :].double() * k[:, :, 0, :].double()).sum(-1)
    assert (lse[:, :, 0].cpu().double() - want).abs().max().item() < 1e-4


@pytest.mark.parametrize("D", [64, 128])
def test_zero_query_uniform(D):
    n = 517
    _, k, v = make_qkv(1, 2, n, D, seed=47)
    q = torch.zeros_like(k)
    o, lse = run(q, k, v, False)
    vf = v.double()
    assert (o.cpu().double() - vf.mean(dim=2, keepdim=True)).abs().max().item() < 1e-2
    assert (lse.cpu().double() - math.log(n)).abs().max().item() < 1e-5
    o, lse = run(q, k, v, True)
    prefix = vf.cumsum(dim=2) / torch.arange(1, n + 1, dtype=torch.float64)[None, None, :, None]
    assert (o.cpu().double() - prefix).abs().max().item() < 1e-2
    want = torch.log(torch.arange(1, n + 1, dtype=torch.float64))
    assert (lse.cpu().double() - want).abs().max().item() < 1e-5


# ---------------------------------------------------------------- memory behaviour

@pytest.mark.parametrize("N,D,causal", [(1, 64, False), (130, 128, True), (301, 64, False)])
def test_writes_every_row_and_nothing_else(N, D, causal):
    """Outputs start as NaN inside guard bands of canary values; every row must be written
    and no byte outside the output must change."""
    dev = torch.device("cuda:0")
    B, H, G = 2, 3, 256
    q, k, v = make_qkv(B, H, N, D, seed=53)
    n_o, n_l = B * H * N * D, B * H * N
    o_buf = torch.full((n_o + 2 * G,), float("nan"), dtype=torch.bfloat16, device=dev)
    l_buf = torch.full((n_l + 2 * G,), float("nan"), dtype=torch.float32, device=dev)
    o_buf[:G] = 7.0
    o_buf[-G:] = 7.0
    l_buf[:G] = 7.0
    l_buf[-G:] = 7.0
    o = o_buf[G:G + n_o].view(B, H, N, D)
    lse = l_buf[G:G + n_l].view(B, H, N)
    run(q, k, v, causal, out=o, lse=lse)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "some output rows not written"
    assert (o_buf[:G] == 7.0).all() and (o_buf[-G:] == 7.0).all(), "wrote outside O"
    assert (l_buf[:G] == 7.0).all() and (l_buf[-G:] == 7.0).all(), "wrote outside lse"
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), causal, 1 / math.sqrt(D))
    check(o, lse, o_ref, lse_ref, f"guarded N{N} D{D}")


def test_non_default_stream_and_repeatability():
    q, k, v = make_qkv(2, 4, 640, 128, seed=59)
    o1, l1 = run(q, k, v, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "results must be deterministic"


def test_rejects_bad_arguments_on_gpu():
    q, k, v = (t.cuda() for t in make_qkv(1, 1, 64, 96, seed=1))
    with pytest.raises(ValueError, match="head dimension"):
        attn_fwd(q, k, v)
    q, k, v = (t.cuda() for t in make_qkv(1, 1, 64, 64, seed=1))
    with pytest.raises(ValueError):
        attn_fwd(q, k, v, scale=-1.0)


# ---------------------------------------------------------------- full-size workloads

def sample_rows(w, rng, heads=8, random_rows=8):
    n = w.N
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 129, n // 2, n - 129, n - 128, n - 2, n - 1}
    out = []
    bh = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(heads - 2)]
    bh += [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in bh:
        rows = sorted({i for i in fixed if 0 <= i < n} | set(int(x) for x in rng.integers(0, n, random_rows)))
        out += [(b, h, i) for i in rows]
    return out


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_workload_full_size_sampled(wid):
    w = WORKLOADS[wid]
    print(f"[parity] generating {w.describe()}", flush=True)
    q, k, v = workload_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    # property at any size: lse_i >= any single visible scaled score (here key i)
    diag = w.scale * (qd.float() * kd.float()).sum(-1)
    assert (lse - diag).min().item() >= -1e-3, "lse below a visible score"
    # property at any size: O lies within the per-column range of the visible V rows
    vf = vd.float()
    if w.causal:
        hi = torch.cummax(vf, dim=2).values
        lo = torch.cummin(vf, dim=2).values
    else:
        hi = vf.amax(dim=2, keepdim=True)
        lo = vf.amin(dim=2, keepdim=True)
    of = o.float()
    assert (of - hi).max().item() <= 2e-2 and (lo - of).max().item() <= 2e-2
    del hi, lo, of, vf, diag
    # sampled rows against the per-row oracle
    rng = np.random.default_rng(wid)
    rows = sample_rows(w, rng)
    o_ref = np.empty((len(rows), w.D))
    lse_ref = np.empty(len(rows))
    by_head = {}
    for r, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((r, i))
    for (b, h), items in by_head.items():
        qh, kh, vh = (f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
        ro, rl = oracle.attention_rows(qh, kh, vh, [(0, 0, i) for _, i in items], w.causal, w.scale)
        for (r, _), oo, ll in zip(items, ro, rl):
            o_ref[r], lse_ref[r] = oo, ll
    idx_b = torch.tensor([b for b, _, _ in rows])
    idx_h = torch.tensor([h for _, h, _ in rows])
    idx_i = torch.tensor([i for _, _, i in rows])
    og = o.cpu()[idx_b, idx_h, idx_i]
    lg = lse.cpu()[idx_b, idx_h, idx_i]
    check(og, lg, o_ref, lse_ref, f"{w.describe()} ({len(rows)} sampled rows)")


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_workload_full_size_every_element(wid):
    """The benchmark's launch at full size, compared element by element over the whole
    tensor with the fp64 oracle (run on the host cores, 16 heads at a time)."""
    from threadpoolctl import threadpool_limits

    w = WORKLOADS[wid]
    print(f"[parity] generating {w.describe()}", flush=True)
    q, k, v = workload_inputs(w)
    dev = torch.device("cuda:0")
    o, lse = attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    workers = min(16, len(os.sched_getaffinity(0)))
    qf, kf, vf = (t.view(w.B * w.H, 1, w.N, w.D) for t in (q, k, v))
    of, lf = o.view(w.B * w.H, w.N, w.D), lse.view(w.B * w.H, w.N)
    max_abs = lse_err = 0.0
    diff2 = ref2 = 0.0
    worst = None
    with threadpool_limits(limits=1):
        for h0 in range(0, w.B * w.H, 16):
            h1 = min(w.B * w.H, h0 + 16)
            o_ref, lse_ref = oracle.attention_fwd(f64(qf[h0:h1]).swapaxes(0, 1), f64(kf[h0:h1]).swapaxes(0, 1),
                                                  f64(vf[h0:h1]).swapaxes(0, 1), w.causal, w.scale,
                                                  workers=workers)
            d = f64(of[h0:h1]) - o_ref[0]
            assert np.isfinite(d).all(), "non-finite output"
            per_head = np.abs(d).reshape(h1 - h0, -1).max(axis=1)
            if per_head.max() > max_abs:
                max_abs = float(per_head.max())
                worst = h0 + int(per_head.argmax())
            diff2 += float((d * d).sum())
            ref2 += float((o_ref * o_ref).sum())
            lse_err = max(lse_err, float(np.abs(f64(lf[h0:h1]) - lse_ref[0]).max()))
    rel = math.sqrt(diff2 / ref2)
    print(f"[parity] {w.describe()} (all {w.B * w.H * w.N} rows): O max-abs {max_abs:.3e} "
          f"(worst head {worst}) rel-L2 {rel:.3e} lse max-abs {lse_err:.3e}", flush=True)
    assert max_abs <= O_MAX_ABS and rel <= O_REL_L2 and lse_err <= LSE_MAX_ABS
    if wid == 5:
        # Its peaked rows (scores drawn with sigma 2) leave this workload the least margin:
        # 1.876e-2 against the 2e-2 bar with the kernel's present summation order, the same
        # bits on every device. A change that moves it past 1.9e-2 stops here, before the bar.
        assert max_abs <= 1.9e-2, f"workload 5 O max-abs {max_abs} is closing on the bar"


# ------------------------------------------------------------ sequences of a million keys
LONG = [
    # B, H, N, D, causal: one head of 2^20 keys (causal: the persistent grid of query-tile
    # pairs), a ragged 2^20 - 37 at D = 64 (persistent, two query blocks per wave), and two
    # heads of 2^19 at causal D = 64 (the four-wave kernel)
    (1, 1, 1 << 20, 128, False),
    (1, 1, 1 << 20, 128, True),
    (1, 1, (1 << 20) - 37, 64, False),
    (1, 2, 1 << 19, 64, True),
]


@pytest.mark.parametrize("B,H,N,D,causal", LONG,
                         ids=[f"B{b}H{h}N{n}D{d}{'c' if c else 'n'}" for b, h, n, d, c in LONG])
def test_long_sequence_sampled(B, H, N, D, causal):
    """Sampled rows of sequences far longer than any workload: the fp32 running sum l then
    adds up 2^14 key tiles, and the byte offsets of K, V and O span up to 256 MiB a head."""
    print(f"[parity] long sequence B{B} H{H} N{N} D{D} causal={causal}", flush=True)
    q, k, v = make_qkv(B, H, N, D, seed=4242 + N % 97 + D)
    o, lse = run(q, k, v, causal)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    rng = np.random.default_rng(N + D)
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, 511, 512, N // 2, N - 513, N - 257, N - 256,
             N - 65, N - 64, N - 33, N - 32, N - 2, N - 1]
    rows = []
    for b in range(B):
        for h in range(H):
            picks = sorted({i for i in fixed if 0 <= i < N} | set(int(x) for x in rng.integers(0, N, 6)))
            rows += [(b, h, i) for i in picks]
    o_ref = np.empty((len(rows), D))
    lse_ref = np.empty(len(rows))
    for b in range(B):
        for h in range(H):
            items = [(r, i) for r, (bb, hh, i) in enumerate(rows) if (bb, hh) == (b, h)]
            qh, kh, vh = (f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
            ro, rl = oracle.attention_rows(qh, kh, vh, [(0, 0, i) for _, i in items], causal)
            for (r, _), oo, ll in zip(items, ro, rl):
                o_ref[r], lse_ref[r] = oo, ll
            del qh, kh, vh
    idx = [torch.tensor([x[j] for x in rows]) for j in range(3)]
    check(o.cpu()[idx[0], idx[1], idx[2]], lse.cpu()[idx[0], idx[1], idx[2]], o_ref, lse_ref,
          f"B{B} H{H} N{N} D{D} {'causal' if causal else 'non-causal'} ({len(rows)} sampled rows)")
