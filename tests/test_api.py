"""C-ABI library checks that need no GPU: it loads, exports every declared entry point,
and rejects invalid arguments with the documented codes before any HIP call.

Every call below has at least one invalid argument, so none of them reaches a launch.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from softmax_attention_fwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
HEADER = os.path.join(ROOT, "include", "attn_fwd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from softmax_attention_fwd_amd import build
        build.build()
    return binding.load_library()


def declared_functions(path=None):
    names = set()
    for h in ([path] if path else HEADERS):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def declared_codes(prefix="ATTN_FWD_"):
    text = "".join(open(h).read() for h in HEADERS)
    return {name: int(val) for name, val in re.findall(r"#define\s+(" + prefix + r"\w+)\s+(-?\d+)", text)}


def test_header_declares_entry_points():
    assert declared_functions() == ["attn_bwd", "attn_bwd_strerror", "attn_bwd_workspace_bytes",
                                    "attn_decode", "attn_decode_noalloc", "attn_decode_strerror",
                                    "attn_decode_workspace_bytes", "attn_fwd", "attn_fwd_ex",
                                    "attn_fwd_strerror"]
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "tile_gemm.h")).read(), flags=re.S)
    assert sorted(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(gemm_\w+)\s*\(", text, flags=re.M)) == \
        ["gemm_bf16_nt", "gemm_strerror"]
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "based_fwd.h")).read(), flags=re.S)
    assert sorted(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(based_\w+)\s*\(", text, flags=re.M)) == \
        ["based_fwd", "based_fwd_strerror", "based_fwd_workspace_bytes", "based_fwd_ws"]
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "tile_calibrate.h")).read(), flags=re.S)
    assert sorted(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(tile_\w+)\s*\(", text, flags=re.M)) == \
        ["tile_mfma_calibrate", "tile_mfma_calibrate_out_floats"]


def test_exports_every_declared_symbol(lib):
    import subprocess
    exported = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                              capture_output=True, text=True, check=True).stdout.split()
    for name in declared_functions() + ["gemm_bf16_nt", "gemm_strerror", "based_fwd", "based_fwd_strerror",
                                        "based_fwd_ws", "based_fwd_workspace_bytes",
                                        "tile_mfma_calibrate", "tile_mfma_calibrate_out_floats"]:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
        assert name in exported


def test_kernel_selectors_match_binding():
    assert declared_codes("ATTN_FWD_KERNEL_") == {
        "ATTN_FWD_KERNEL_" + k.upper(): v for k, v in binding.FWD_KERNELS.items()}


def test_codes_match_binding():
    codes = {k: v for k, v in declared_codes().items() if not k.startswith("ATTN_FWD_KERNEL_")}
    assert codes == {
        "ATTN_FWD_OK": binding.ATTN_FWD_OK,
        "ATTN_FWD_EINVAL": binding.ATTN_FWD_EINVAL,
        "ATTN_FWD_EUNSUPPORTED": binding.ATTN_FWD_EUNSUPPORTED,
        "ATTN_FWD_EALIGN": binding.ATTN_FWD_EALIGN,
        "ATTN_FWD_ELAUNCH": binding.ATTN_FWD_ELAUNCH,
    }


def test_bwd_codes_match_binding():
    assert declared_codes("ATTN_BWD_") == {
        "ATTN_BWD_OK": 0, "ATTN_BWD_EINVAL": binding.ATTN_FWD_EINVAL,
        "ATTN_BWD_EUNSUPPORTED": binding.ATTN_FWD_EUNSUPPORTED,
        "ATTN_BWD_EALIGN": binding.ATTN_FWD_EALIGN, "ATTN_BWD_ELAUNCH": binding.ATTN_FWD_ELAUNCH,
        "ATTN_BWD_EWORKSPACE": binding.ATTN_BWD_EWORKSPACE,
    }


def test_bwd_strerror(lib):
    msgs = {lib.attn_bwd_strerror(c).decode() for c in declared_codes("ATTN_BWD_").values()}
    assert len(msgs) == len(declared_codes("ATTN_BWD_")) and "unknown error code" not in msgs


def test_strerror(lib):
    seen = set()
    codes = {k: v for k, v in declared_codes().items() if not k.startswith("ATTN_FWD_KERNEL_")}
    for code in codes.values():
        msg = lib.attn_fwd_strerror(code).decode()
        assert msg and msg != "unknown error code"
        seen.add(msg)
    assert len(seen) == len(codes)
    assert lib.attn_fwd_strerror(12345).decode() == "unknown error code"


# Fake, never-dereferenced addresses: validation returns before touching them.
A = 0x10000  # 16-byte aligned


def call(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=128, D=64, causal=0, scale=0.125):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, D, causal, ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1),
    (dict(B=0), -1), (dict(H=0), -1), (dict(N=0), -1), (dict(N=-5), -1),
    (dict(causal=2), -1), (dict(causal=-1), -1),
    (dict(scale=0.0), -1), (dict(scale=-1.0), -1), (dict(scale=math.inf), -1),
    (dict(scale=math.nan), -1),
    (dict(D=96), -2), (dict(D=32), -2), (dict(D=256), -2), (dict(D=0), -2),
    (dict(N=1 << 24, D=128), -1),                   # N*D reaches 2^31
    (dict(B=1 << 16, H=1 << 16, N=1 << 10), -1),    # grid reaches 2^31 workgroups
    (dict(q=A + 8), -3), (dict(k=A + 2), -3), (dict(v=A + 4), -3), (dict(o=A + 1), -3),
    (dict(lse=A + 2), -3),
])
def test_invalid_arguments_rejected(lib, kw, code):
    assert call(lib, **kw) == code


@pytest.mark.parametrize("kernel,code", [(3, -1), (-1, -1), (1, -2), (2, -2)])
def test_fwd_ex_rejects_bad_kernel_and_shape(lib, kernel, code):
    # an unknown selector is EINVAL; a valid one still validates the rest (D = 96 here)
    D = 96 if code == -2 else 64
    assert lib.attn_fwd_ex(A, A, A, A, A, 1, 1, 128, D, 0, ctypes.c_float(0.125), kernel, None) == code


def test_binding_rejects_cpu_and_bad_dtypes():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        binding.attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="bfloat16"):
        binding.attn_fwd(q.float(), q, q)
    with pytest.raises(ValueError, match="shape"):
        binding.attn_fwd(q[0], q, q)
    with pytest.raises(ValueError, match="contiguous"):
        binding.attn_fwd(q.transpose(2, 3), q, q)


def test_binding_missing_library_is_loud(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setenv("ATTN_FWD_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library()


def test_bwd_workspace_bytes(lib):
    # two fp32 arrays of B*H*N, each rounded up to 256 bytes
    assert lib.attn_bwd_workspace_bytes(2, 3, 100) == 2 * 2560
    assert lib.attn_bwd_workspace_bytes(16, 16, 4096) == 2 * 16 * 16 * 4096 * 4
    assert lib.attn_bwd_workspace_bytes(0, 1, 1) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, -3) == 0


W = 0x100000  # 256-byte aligned fake workspace


def call_bwd(lib, q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, ws=W, ws_bytes=1 << 20,
             B=1, H=1, N=128, D=64, causal=0, scale=0.125):
    return lib.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, N, D, causal,
                        ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(do=None), -1), (dict(lse=None), -1),
    (dict(dq=None), -1), (dict(dv=None), -1), (dict(ws=None), -1),
    (dict(B=0), -1), (dict(N=0), -1), (dict(causal=3), -1), (dict(scale=-2.0), -1),
    (dict(scale=math.nan), -1), (dict(D=80), -2), (dict(N=1 << 24, D=128), -1),
    (dict(ws_bytes=100), -5), (dict(B=16, H=16, N=4096, ws_bytes=1 << 20), -5),
    (dict(do=A + 4), -3), (dict(dk=A + 2), -3), (dict(lse=A + 1), -3), (dict(ws=W + 16), -3),
])
def test_bwd_invalid_arguments_rejected(lib, kw, code):
    assert call_bwd(lib, **kw) == code


def test_bwd_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError, match="GPU"):
        binding.attn_bwd(q, q, q, q, q, lse)


def test_decode_codes_and_strerror(lib):
    codes = declared_codes("ATTN_DECODE_")
    assert codes == {"ATTN_DECODE_OK": 0, "ATTN_DECODE_EINVAL": -1, "ATTN_DECODE_EUNSUPPORTED": -2,
                     "ATTN_DECODE_EALIGN": -3, "ATTN_DECODE_ELAUNCH": -4, "ATTN_DECODE_EWORKSPACE": -5}
    msgs = {lib.attn_decode_strerror(c).decode() for c in codes.values()}
    assert len(msgs) == len(codes) and "unknown error code" not in msgs


def test_decode_workspace_bytes(lib):
    # about one workgroup per compute unit (256): 256 heads -> one key chunk each; partial
    # O (fp32) and lse per chunk and query, each array rounded up to 256 bytes
    assert lib.attn_decode_workspace_bytes(16, 16, 1, 4096, 128) == 1 * 256 * 128 * 4 + 1024
    # 8 heads -> 32 chunks of 128 keys each
    assert lib.attn_decode_workspace_bytes(1, 8, 1, 4096, 128) == 32 * 8 * 128 * 4 + 1024
    # 4 heads of 200 keys -> at most ceil(200 / 128) = 2 chunks; 3 queries
    assert lib.attn_decode_workspace_bytes(2, 2, 3, 200, 64) == 2 * 4 * 3 * 64 * 4 + 256
    assert lib.attn_decode_workspace_bytes(1, 1, 33, 100, 64) == 0   # Nq > 32
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 100, 96) == 0    # unsupported D
    assert lib.attn_decode_workspace_bytes(0, 1, 1, 100, 64) == 0


def call_dec(lib, q=A, k=A, v=A, o=A, lse=A, ws=W, ws_bytes=1 << 24, B=1, H=1, Nq=1, Nk=128,
             D=64, causal=0, scale=0.125):
    return lib.attn_decode(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, D, causal,
                           ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(lse=None), -1), (dict(ws=None), -1),
    (dict(Nq=0), -1), (dict(Nk=0), -1), (dict(B=0), -1), (dict(causal=2), -1),
    (dict(causal=1, Nq=8, Nk=4), -1), (dict(scale=0.0), -1), (dict(scale=math.inf), -1),
    (dict(D=96), -2), (dict(Nq=33), -2), (dict(Nk=1 << 24, D=128), -1),
    (dict(ws_bytes=10), -5), (dict(q=A + 8), -3), (dict(o=A + 2), -3), (dict(lse=A + 1), -3),
    (dict(ws=W + 64), -3),
])
def test_decode_invalid_arguments_rejected(lib, kw, code):
    assert call_dec(lib, **kw) == code


def call_dec_noalloc(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=1, Nk=128, D=64, causal=0,
                     scale=0.125):
    return lib.attn_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, causal, ctypes.c_float(scale), None)


NOALLOC_MAX = 33 << 20  # ATTN_DECODE_NOALLOC_MAX_WORKSPACE


def test_decode_noalloc_limit_declared():
    text = open(os.path.join(ROOT, "include", "attn_decode.h")).read()
    m = re.search(r"#define\s+ATTN_DECODE_NOALLOC_MAX_WORKSPACE\s+\(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == NOALLOC_MAX


def test_decode_noalloc_limit_covers_up_to_1024_heads(lib):
    # the chunk plan keeps B*H*S below 1024 + B*H, so 32 queries of D = 128 fit for B*H <= 1024
    for bh in (1, 7, 256, 1000, 1024):
        for nk in (1, 129, 4096, 131072, (1 << 24) - 1):
            assert 0 < lib.attn_decode_workspace_bytes(1, bh, 32, nk, 128) <= NOALLOC_MAX
    assert lib.attn_decode_workspace_bytes(64, 64, 32, 256, 128) > NOALLOC_MAX


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(Nq=0), -1), (dict(B=0), -1),
    (dict(causal=2), -1), (dict(causal=1, Nq=8, Nk=4), -1), (dict(scale=-1.0), -1),
    (dict(D=96), -2), (dict(Nq=33), -2),
    (dict(B=64, H=64, Nq=32, Nk=256, D=128), -5),   # partials beyond the fixed scratch
    (dict(q=A + 8), -3), (dict(lse=A + 1), -3),
])
def test_decode_noalloc_invalid_arguments_rejected(lib, kw, code):
    assert call_dec_noalloc(lib, **kw) == code


def test_gemm_codes_and_strerror(lib):
    text = open(os.path.join(ROOT, "include", "tile_gemm.h")).read()
    codes = {n: int(v) for n, v in re.findall(r"#define\s+(GEMM_\w+)\s+(-?\d+)", text)}
    assert codes == {"GEMM_OK": 0, "GEMM_EINVAL": -1, "GEMM_EALIGN": -3, "GEMM_ELAUNCH": -4}
    msgs = {lib.gemm_strerror(c).decode() for c in codes.values()}
    assert len(msgs) == len(codes) and "unknown error code" not in msgs


@pytest.mark.parametrize("args,code", [
    ((None, A, A, 8, 8, 8), -1), ((A, None, A, 8, 8, 8), -1), ((A, A, None, 8, 8, 8), -1),
    ((A, A, A, 0, 8, 8), -1), ((A, A, A, 8, 0, 8), -1), ((A, A, A, 8, 8, 0), -1),
    ((A, A, A, 8, 8, 12), -1), ((A, A, A, 8, 12, 8), -1), ((A, A, A, 1 << 20, 8, 1 << 10), -1),
    ((A + 8, A, A, 8, 8, 8), -3), ((A, A + 2, A, 8, 8, 8), -3), ((A, A, A + 4, 8, 8, 8), -3),
])
def test_gemm_invalid_arguments_rejected(lib, args, code):
    assert lib.gemm_bf16_nt(*args, None) == code


def test_based_codes_and_strerror(lib):
    text = open(os.path.join(ROOT, "include", "based_fwd.h")).read()
    codes = {n: int(v) for n, v in re.findall(r"#define\s+(BASED_\w+)\s+(-?\d+)", text)}
    assert codes == {"BASED_OK": 0, "BASED_EINVAL": -1, "BASED_EUNSUPPORTED": -2, "BASED_EALIGN": -3,
                     "BASED_ELAUNCH": -4}
    msgs = {lib.based_fwd_strerror(c).decode() for c in codes.values()}
    assert len(msgs) == len(codes) and "unknown error code" not in msgs


@pytest.mark.parametrize("args,code", [
    ((None, A, A, A, 1, 1, 64, 16, 64), -1), ((A, None, A, A, 1, 1, 64, 16, 64), -1),
    ((A, A, None, A, 1, 1, 64, 16, 64), -1), ((A, A, A, None, 1, 1, 64, 16, 64), -1),
    ((A, A, A, A, 0, 1, 64, 16, 64), -1), ((A, A, A, A, 1, 0, 64, 16, 64), -1),
    ((A, A, A, A, 1, 1, 0, 16, 64), -1), ((A, A, A, A, 1, 1, 1 << 24, 16, 64), -1),
    ((A, A, A, A, 1, 1, 64, 32, 64), -2), ((A, A, A, A, 1, 1, 64, 16, 128), -2),
    ((A + 8, A, A, A, 1, 1, 64, 16, 64), -3), ((A, A, A + 2, A, 1, 1, 64, 16, 64), -3),
    ((A, A, A, A + 4, 1, 1, 64, 16, 64), -3),
])
def test_based_invalid_arguments_rejected(lib, args, code):
    assert lib.based_fwd(*args, None) == code


def test_based_ws_checks_before_any_device_query(lib):
    assert lib.based_fwd_ws(A, A, A, A, A + 16, 1 << 20, 1, 1, 64, 16, 64, None) == -3
    assert lib.based_fwd_ws(None, A, A, A, None, 0, 1, 1, 64, 16, 64, None) == -1
    assert lib.based_fwd_ws(A, A, A, A, None, 0, 1 << 12, 1 << 12, 64, 16, 64, None) == -1
    assert lib.based_fwd_ws(A, A, A, A, None, 0, 1, 1, 64, 16, 32, None) == -2
    assert lib.based_fwd_workspace_bytes(0, 1, 64) == 0
    assert lib.based_fwd_workspace_bytes(1, 1, 0) == 0


def test_based_binding_rejects_cpu_and_bad_shapes():
    import torch
    from softmax_attention_fwd_amd import based_fwd
    q = torch.zeros(1, 1, 8, 16, dtype=torch.bfloat16)
    v = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        based_fwd(q, q, v)
    with pytest.raises(ValueError, match="bfloat16"):
        based_fwd(q.float(), q, v)
    with pytest.raises(TypeError):
        based_fwd(q.numpy(), q, v)


def test_mfma_calibrate_rejects_bad_arguments(lib):
    # argument checks that come before any device query
    flops = ctypes.c_double(0.0)
    assert lib.tile_mfma_calibrate(None, 1 << 20, 10, 1, ctypes.byref(flops), None) == -1
    assert lib.tile_mfma_calibrate(A, 1 << 20, 0, 1, ctypes.byref(flops), None) == -1
    assert lib.tile_mfma_calibrate(A, 1 << 20, 10, 2, ctypes.byref(flops), None) == -1
    assert lib.tile_mfma_calibrate(A, 1 << 20, (1 << 24) + 1, 0, ctypes.byref(flops), None) == -1
    assert lib.tile_mfma_calibrate(A, 1 << 20, 10, 0, None, None) == -1
