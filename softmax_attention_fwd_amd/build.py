"""Build ``libattn_fwd.so`` in-tree with hipcc for gfx950.

    python -m softmax_attention_fwd_amd.build        # or __graft_entry__.build()

The library holds six translation units, each with its kernels and C entry points:
csrc/attn_fwd.hip (the forward), csrc/attn_bwd.hip (the backward),
csrc/attn_decode.hip (the decode-shaped split-KV forward), csrc/gemm.hip (the plain
bf16 matrix product on the same tile layer), csrc/based_fwd.hip (Based linear
attention) and csrc/calibrate.hip (the sustained matrix-core rate probe that bench.py
reads measured rates against). It is built for
gfx950 only, with packed fp32 VALU instructions disabled (the compiler would otherwise
form v_pk_* fp32 ops from plain float code).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "gemm.hip",
                                                 "based_fwd.hip", "calibrate.hip")]
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libattn_fwd.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile the library (always, even if a build exists) and return its path."""
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx950 feature flag and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv[1:]))
