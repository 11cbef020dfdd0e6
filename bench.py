#!/usr/bin/env python3
"""Attention forward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--gpus 1]
                    [--op fwd|bwd|decode|gemm|based]

One step = one attn_fwd call (the whole fused forward: K/V streaming, both contractions,
online softmax, epilogue) over the workload's full tensors, already resident in HBM; with
--op bwd, one attn_bwd call (its kernels: Delta, dK/dV, dQ) on the same shapes; with
--op decode, one attn_decode call (split kernel + merge) on a decode workload (1..3:
few queries against a long KV cache), reported in GB/s of K and V read against HBM; with
--op gemm, one C = A B^T (bf16) of --gemm-shape M,N,K, in TFLOP/s (2*M*N*K); with
--op based, one based_fwd call (Based linear attention, causal, d = 16, dv = 64) on a
Based workload (1..3, default 2: B16 H16 N4096), in GB/s of q, k, v, o against HBM.
The default workload is B16 H16 N4096 D128 non-causal with bf16 inputs. Prints ONE JSON
line on stdout; details go to stderr.

Reported:
  value          whole-job TFLOP/s = F * K / (timed span), with F = 4*B*H*N^2*D for the
                 forward and 10*B*H*N^2*D for the backward (its five N x N x D products),
                 halved when causal
  roofline       F over the mean duration of one call (HIP events on the launch stream)
                 against the bf16 dense MFMA peak
  cpu_baseline   the fp64 numpy oracle of the same pass, timed on this host's cores on a
                 bounded sample of the same workload (a few heads), in the same unit, with
                 the threads it used ("cores") and the host CPU's model name ("cpu")
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X bf16 dense MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "softmax_attention_fwd_amd", "csrc", "attn_fwd.hip")

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (separate
# runs), scaled by what the same counters read for a 512 MiB device-to-device copy: FETCH_SIZE
# reported 262157.6 KiB for 524288 KiB read (x 2.0), WRITE_SIZE 524288 KiB for 524288 KiB
# written (x 1.0). Valid only for the kernel source they were taken on; any other source
# reports null.
MEASURED_TRAFFIC = {
    "w3_b16h16n4096d128": {
        "source_sha256": "5e85cb7032bba45fa54275db1c84a311bc9d3da3b57af42a824c0a31fd7c88f5",
        "fetch_kib": 393426.1 * 2.0,
        "write_kib": 266829.6 * 1.0,
    },
    "w2_b16h16n1024d64": {
        "source_sha256": "5e85cb7032bba45fa54275db1c84a311bc9d3da3b57af42a824c0a31fd7c88f5",
        "fetch_kib": 49370.0 * 2.0,
        "write_kib": 33795.8 * 1.0,
    },
}


def source_digest() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload_name: str):
    m = MEASURED_TRAFFIC.get(workload_name)
    if m is None or m["source_sha256"] != source_digest():
        return None
    return int(round((m["fetch_kib"] + m["write_kib"]) * 1024))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" where it cannot be read)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def mfma_sustained(stream, iterations: int = 25000, reps: int = 4):
    """Rates of the sustained matrix-core probe (include/tile_calibrate.h): the best of
    ``reps`` runs with zero operands and with random bf16 operands, each ~25 ms."""
    import torch

    from softmax_attention_fwd_amd import mfma_calibrate
    rates = {}
    for random_operands in (False, True):
        best = 0.0
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            flops = mfma_calibrate(iterations, random_operands, stream=stream)
            e1.record(stream)
            e1.synchronize()
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        key = "random_tflops" if random_operands else "zeros_tflops"
        rates[key] = round(best, 1)
        log(f"[bench] sustained MFMA probe, {'random' if random_operands else 'zero'} operands: "
            f"{best:.1f} TFLOP/s ({100 * best / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS})")
    rates["peak_frac_random"] = round(rates["random_tflops"] / PEAK_BF16_TFLOPS, 4)
    return rates


def cpu_baseline(w, q, k, v, budget_s: float, do=None):
    """Time the fp64 oracle (forward, or backward when ``do`` is given) on whole heads of
    the workload, one head per host core."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    per_head = (w.flops if do is None else 2.5 * w.flops) / (w.B * w.H)
    heads = min(w.B * w.H, cores)
    b_idx = [i // w.H for i in range(heads)]
    h_idx = [i % w.H for i in range(heads)]
    qs = np.stack([q[b, h].double().numpy() for b, h in zip(b_idx, h_idx)])[None]
    ks = np.stack([k[b, h].double().numpy() for b, h in zip(b_idx, h_idx)])[None]
    vs = np.stack([v[b, h].double().numpy() for b, h in zip(b_idx, h_idx)])[None]
    if do is not None:
        dos = np.stack([do[b, h].double().numpy() for b, h in zip(b_idx, h_idx)])[None]
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        done = 0
        t0 = time.perf_counter()
        while True:
            if do is None:
                oracle.attention_fwd(qs, ks, vs, w.causal, w.scale, workers=cores)
            else:
                oracle.attention_bwd(qs, ks, vs, dos, w.causal, w.scale, workers=cores)
            done += heads
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {
        "value": round(done * per_head / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores, "cpu": cpu_model(),
        "kind": "oracle",
        "sample": (f"{done} head-passes ({'forward' if do is None else 'backward'}) of "
                   f"{w.describe()} (first {heads} heads, "
                   f"{done * per_head:.3e} flop, fp64 numpy, one head per thread) in {dt:.1f} s"),
    }


def time_steps(step, stream, steps: int, warmup: int):
    """Run warmup steps, then time `steps` steps with per-step HIP events and one span
    pair on `stream`. Returns (span_ms, per-step ms list, wall seconds)."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup} done; timing {steps} steps")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    span0 = torch.cuda.Event(enable_timing=True)
    span1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    span0.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    span1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return span0.elapsed_time(span1), [a.elapsed_time(b) for a, b in zip(starts, ends)], wall


def decode_cpu_baseline(w, q, k, v, budget_s: float):
    """Time the fp64 decode oracle on whole heads, one head per host core, in GB/s of the
    workload's algorithmic bytes per head."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    nh = w.B * w.H
    heads = min(nh, cores)
    per_head = w.hbm_bytes / nh
    qs = [q.view(nh, 1, 1, w.Nq, w.D)[i].double().numpy() for i in range(heads)]
    ks = [k.view(nh, 1, 1, w.Nk, w.D)[i].double().numpy() for i in range(heads)]
    vs = [v.view(nh, 1, 1, w.Nk, w.D)[i].double().numpy() for i in range(heads)]
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        done = 0
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=heads) as ex:
            while True:
                list(ex.map(lambda i: oracle.attention_decode(qs[i], ks[i], vs[i], w.causal, w.scale),
                            range(heads)))
                done += heads
                if time.perf_counter() - t0 >= budget_s:
                    break
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {
        "value": round(done * per_head / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores, "cpu": cpu_model(),
        "kind": "oracle",
        "sample": (f"{done} head-passes (decode) of {w.describe()} (first {heads} heads, "
                   f"{done * per_head / 1e9:.3f} GB of K/V/Q/O, fp64 numpy, one head per thread) "
                   f"in {dt:.1f} s"),
    }


def run_decode(args) -> int:
    import torch

    from softmax_attention_fwd_amd import attn_decode, decode_workspace_bytes
    from softmax_attention_fwd_amd.inputs import DECODE_WORKLOADS, decode_inputs

    w = DECODE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] decode workload {args.workload}: {w.describe()}; generating inputs (seed {w.seed})")
    q, k, v = decode_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(decode_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        attn_decode(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws,
                    stream=stream)

    total_ms, launch_ms, wall = time_steps(step, stream, args.steps, args.warmup)
    mean_launch = statistics.fmean(launch_ms)
    value = w.hbm_bytes * args.steps / (total_ms * 1e-3) / 1e9
    achieved = w.hbm_bytes / (mean_launch * 1e-3) / 1e9
    log(f"[bench] span {total_ms:.3f} ms for {args.steps} steps; launch median "
        f"{statistics.median(launch_ms):.4f} ms; {value:.1f} GB/s whole-job, {achieved:.1f} GB/s "
        f"per call = {100 * achieved / PEAK_HBM_GBS:.1f}% of HBM peak")
    result = {
        "metric": "attention decode (split-KV) GB/s of K, V, Q, O and lse against HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q, K, V)",
        "config": {"workload": w.name, "op": "decode", "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk,
                   "D": w.D, "causal": w.causal, "scale": w.scale, "parallelism": "single GPU"},
        "launch_ms": {"mean": round(mean_launch, 5), "median": round(statistics.median(launch_ms), 5),
                      "min": round(min(launch_ms), 5), "max": round(max(launch_ms), 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "traffic_algorithmic": w.hbm_bytes},
        "cpu_baseline": None,
    }
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 512 MiB device-to-device")
        del src, dst
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 decode oracle on host cores (~{args.cpu_seconds:.0f} s budget)")
        result["cpu_baseline"] = decode_cpu_baseline(w, q, k, v, args.cpu_seconds)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


def run_gemm(args) -> int:
    import torch

    from softmax_attention_fwd_amd import gemm_nt

    M, N, K = (int(x) for x in args.gemm_shape.split(","))
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(3001)
    a = torch.randn((M, K), generator=g).to(torch.bfloat16)
    b = torch.randn((N, K), generator=g).to(torch.bfloat16)
    ad, bd = a.to(dev), b.to(dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = 2.0 * M * N * K
    log(f"[bench] gemm C = A B^T, M {M} N {N} K {K} (bf16, seed 3001)")

    def step():
        gemm_nt(ad, bd, out=c, stream=stream)

    total_ms, launch_ms, wall = time_steps(step, stream, args.steps, args.warmup)
    mean_launch = statistics.fmean(launch_ms)
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flops / (mean_launch * 1e-3) / 1e12
    log(f"[bench] {value:.1f} TFLOP/s whole-job; kernel {achieved:.1f} TFLOP/s = "
        f"{100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 dense peak")
    result = {
        "metric": "bf16 GEMM C = A B^T TFLOP/s (2*M*N*K) and % of bf16 MFMA peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 A, B)",
        "config": {"workload": f"gemm_m{M}n{N}k{K}", "op": "gemm", "M": M, "N": N, "K": K,
                   "parallelism": "single GPU"},
        "launch_ms": {"mean": round(mean_launch, 5), "median": round(statistics.median(launch_ms), 5),
                      "min": round(min(launch_ms), 5), "max": round(max(launch_ms), 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "traffic_algorithmic": 2 * (M * K + N * K + M * N)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle
        cores = len(os.sched_getaffinity(0))
        rows = max(1, min(M, 256))
        an, bn = a[:rows].double().numpy(), b.double().numpy()
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.gemm_nt(an, bn)
            done += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(done * 2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} products of the first {rows} rows of A with B (fp64 numpy, BLAS threads "
                      f"as numpy sets them) in {dt:.1f} s"}
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


def run_based(args) -> int:
    import torch

    from softmax_attention_fwd_amd import based_fwd
    from softmax_attention_fwd_amd.inputs import BASED_WORKLOADS, based_inputs

    w = BASED_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] based workload: {w.describe()}; generating inputs (seed {w.seed})")
    q, k, v = based_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(vd)
    stream = torch.cuda.current_stream(dev)
    from softmax_attention_fwd_amd.binding import based_fwd_workspace_bytes
    need = based_fwd_workspace_bytes(w.B, w.H, w.N)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None
    if need > 0:
        log(f"[bench] split launch: {need / 2**20:.1f} MiB of segment states")

    def step():
        based_fwd(qd, kd, vd, out=o, workspace=ws, stream=stream)

    total_ms, launch_ms, wall = time_steps(step, stream, args.steps, args.warmup)
    mean_launch = statistics.fmean(launch_ms)
    value = w.hbm_bytes * args.steps / (total_ms * 1e-3) / 1e9
    achieved = w.hbm_bytes / (mean_launch * 1e-3) / 1e9
    tflops = w.flops / (mean_launch * 1e-3) / 1e12
    log(f"[bench] span {total_ms:.3f} ms for {args.steps} steps; launch median "
        f"{statistics.median(launch_ms):.4f} ms; {achieved:.1f} GB/s = "
        f"{100 * achieved / PEAK_HBM_GBS:.1f}% of HBM peak; {tflops:.1f} TFLOP/s of the chunked form")
    result = {
        "metric": "Based linear attention fwd (causal) GB/s of q, k, v, o against HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q, k, v)",
        "config": {"workload": w.name, "op": "based", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "dv": w.dv, "causal": True, "parallelism": "single GPU"},
        "launch_ms": {"mean": round(mean_launch, 5), "median": round(statistics.median(launch_ms), 5),
                      "min": round(min(launch_ms), 5), "max": round(max(launch_ms), 5)},
        "tflops_chunked_form": round(tflops, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "traffic_algorithmic": w.hbm_bytes},
        "cpu_baseline": None,
    }
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 512 MiB device-to-device")
        del src, dst
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle
        cores = len(os.sched_getaffinity(0))
        per_head = w.hbm_bytes / (w.B * w.H)
        qn, kn, vn = (t.double().numpy() for t in (q, k, v))
        done, t0 = 0, time.perf_counter()
        while True:
            b, h = divmod(done % (w.B * w.H), w.H)
            oracle.based_linear_attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1])
            done += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(done * per_head / dt / 1e9, 6), "unit": "GB/s", "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} heads of {w.describe()} by the quadratic definition (fp64 numpy, BLAS "
                      f"threads as numpy sets them) in {dt:.1f} s"}
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed launches first; the shader clock settles over ~20 launches")
    ap.add_argument("--workload", type=int, default=None,
                    help="fwd/bwd 1..5, decode 1..3 (default 3); based 1..3 (default 2)")
    ap.add_argument("--op", choices=("fwd", "bwd", "decode", "gemm", "based"), default="fwd",
                    help="the forward (default, the headline metric), the backward pass, or "
                         "the decode-shaped split-KV forward, the plain GEMM, or Based linear "
                         "attention")
    ap.add_argument("--gemm-shape", default="8192,8192,8192", help="M,N,K for --op gemm")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device-to-device copy (3 times) so that "
                         "hardware byte counters can be scaled against a kernel of known traffic")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="after the timed steps, run the sustained matrix-core probe (4 x ~25 ms "
                         "with zero operands, then 4 with random bf16 operands) and report its "
                         "rates under \"mfma_sustained\"")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention forward runs on a single MI355X "
              "and the library has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    if args.op == "decode":
        return run_decode(args)
    if args.workload is None:
        args.workload = 2 if args.op == "based" else 3
    if args.op == "based":
        return run_based(args)
    if args.op == "gemm":
        return run_gemm(args)

    import torch

    from softmax_attention_fwd_amd import attn_bwd, attn_fwd, bwd_workspace_bytes
    from softmax_attention_fwd_amd.inputs import WORKLOADS, make_dout, workload_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] device {props.name} ({props.gcnArchName}), {props.multi_processor_count} CUs")
    log(f"[bench] workload {args.workload}: {w.describe()}; generating inputs (seed {w.seed})")
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    flops = w.flops
    do = None
    if args.op == "fwd":
        def step():
            attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
    else:
        flops = 2.5 * w.flops
        do = make_dout(w.B, w.H, w.N, w.D, seed=w.seed)
        dod = do.to(dev)
        attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        grads = [torch.empty_like(qd) for _ in range(3)]
        ws = torch.empty(bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)

        def step():
            attn_bwd(qd, kd, vd, o, dod, lse, causal=w.causal, scale=w.scale, dq=grads[0],
                     dk=grads[1], dv=grads[2], workspace=ws, stream=stream)

    total_ms, launch_ms, wall = time_steps(step, stream, args.steps, args.warmup)
    mean_launch = statistics.fmean(launch_ms)
    ms_per_step = total_ms / args.steps
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flops / (mean_launch * 1e-3) / 1e12
    log(f"[bench] span {total_ms:.3f} ms for {args.steps} steps ({ms_per_step:.4f} ms/step, "
        f"wall {wall * 1e3:.1f} ms); launch median {statistics.median(launch_ms):.4f} "
        f"min {min(launch_ms):.4f} max {max(launch_ms):.4f} ms")
    log(f"[bench] {value:.1f} TFLOP/s whole-job; kernel {achieved:.1f} TFLOP/s = "
        f"{100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 dense peak")

    metric = "attention fwd TFLOP/s and % of bf16 MFMA peak (B16 H16 N4096 D128)"
    if args.op == "bwd":
        metric = "attention bwd TFLOP/s (10*B*H*N^2*D, halved causal) and % of bf16 MFMA peak"
    result = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q, K, V)",
        "config": {"workload": w.name, "op": args.op, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "launch_ms": {"mean": round(mean_launch, 5), "median": round(statistics.median(launch_ms), 5),
                      "min": round(min(launch_ms), 5), "max": round(max(launch_ms), 5)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name) if args.op == "fwd" else None,
            "traffic_algorithmic": w.hbm_bytes if args.op == "fwd" else 16 * w.B * w.H * w.N * w.D + 12 * w.B * w.H * w.N,
        },
        "cpu_baseline": None,
    }
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 512 MiB device-to-device")
        del src, dst
    if args.calibrate_mfma:
        result["mfma_sustained"] = mfma_sustained(stream)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on host cores (~{args.cpu_seconds:.0f} s budget)")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, do=do)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
