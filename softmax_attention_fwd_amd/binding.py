"""Python binding of the C-ABI attention library (``libattn_fwd.so``).

Argument marshalling only: shapes, dtypes and devices are checked, output tensors are
allocated with torch when the caller gives none, and the C entry point is called with raw
device pointers and the current HIP stream. Every step of the computation runs in the
library's HIP kernels; if the library is missing this module raises instead of computing
anything itself.

C entry points (declared in include/attn_fwd.h, attn_bwd.h, attn_decode.h, tile_gemm.h,
based_fwd.h, tile_calibrate.h):
  int attn_fwd(q, k, v, o, lse, B, H, N, D, causal, scale, stream)
  int attn_fwd_ex(q, k, v, o, lse, B, H, N, D, causal, scale, kernel, stream)
  const char* attn_fwd_strerror(int code)
  size_t attn_bwd_workspace_bytes(B, H, N)
  int attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
               B, H, N, D, causal, scale, stream)
  const char* attn_bwd_strerror(int code)
  size_t attn_decode_workspace_bytes(B, H, Nq, Nk, D)
  int attn_decode(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, D, causal,
                  scale, stream)
  int attn_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale, stream)
  const char* attn_decode_strerror(int code)
  int gemm_bf16_nt(a, b, c, M, N, K, stream)
  const char* gemm_strerror(int code)
  int based_fwd(q, k, v, o, B, H, N, D, F, stream)
  size_t based_fwd_workspace_bytes(B, H, N)
  int based_fwd_ws(q, k, v, o, workspace, workspace_bytes, B, H, N, D, F, stream)
  const char* based_fwd_strerror(int code)
  size_t tile_mfma_calibrate_out_floats(void)
  int tile_mfma_calibrate(out, out_floats, iterations, random_operands, flops, stream)
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn_fwd.so"

# Return codes of the C ABI (mirrors include/attn_fwd.h).
ATTN_FWD_OK = 0
ATTN_FWD_EINVAL = -1
ATTN_FWD_EUNSUPPORTED = -2
ATTN_FWD_EALIGN = -3
ATTN_FWD_ELAUNCH = -4
ATTN_BWD_EWORKSPACE = -5

# Kernel selectors of attn_fwd_ex (include/attn_fwd.h).
FWD_KERNELS = {"auto": 0, "pingpong": 1, "fourwave": 2}

_lock = threading.Lock()
_lib = None


class AttnFwdError(RuntimeError):
    """A nonzero return code from the C entry point."""

    def __init__(self, code: int, message: str):
        super().__init__(f"attn_fwd failed with code {code}: {message}")
        self.code = code


def library_path() -> str:
    return os.environ.get("ATTN_FWD_LIB", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load ``libattn_fwd.so`` once and declare the C signatures. Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, vp]
        lib.attn_fwd.restype = ci
        lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp]
        lib.attn_fwd_ex.restype = ci
        lib.attn_fwd_strerror.argtypes = [ci]
        lib.attn_fwd_strerror.restype = ctypes.c_char_p
        sz = ctypes.c_size_t
        lib.attn_bwd_workspace_bytes.argtypes = [ci, ci, ci]
        lib.attn_bwd_workspace_bytes.restype = sz
        lib.attn_bwd.argtypes = [vp] * 10 + [sz] + [ci] * 5 + [ctypes.c_float, vp]
        lib.attn_bwd.restype = ci
        lib.attn_bwd_strerror.argtypes = [ci]
        lib.attn_bwd_strerror.restype = ctypes.c_char_p
        lib.attn_decode_workspace_bytes.argtypes = [ci] * 5
        lib.attn_decode_workspace_bytes.restype = sz
        lib.attn_decode.argtypes = [vp] * 6 + [sz] + [ci] * 6 + [ctypes.c_float, vp]
        lib.attn_decode.restype = ci
        lib.attn_decode_noalloc.argtypes = [vp] * 5 + [ci] * 6 + [ctypes.c_float, vp]
        lib.attn_decode_noalloc.restype = ci
        lib.attn_decode_strerror.argtypes = [ci]
        lib.attn_decode_strerror.restype = ctypes.c_char_p
        lib.gemm_bf16_nt.argtypes = [vp, vp, vp, ci, ci, ci, vp]
        lib.gemm_bf16_nt.restype = ci
        lib.gemm_strerror.argtypes = [ci]
        lib.gemm_strerror.restype = ctypes.c_char_p
        lib.based_fwd.argtypes = [vp] * 4 + [ci] * 5 + [vp]
        lib.based_fwd.restype = ci
        lib.based_fwd_workspace_bytes.argtypes = [ci, ci, ci]
        lib.based_fwd_workspace_bytes.restype = sz
        lib.based_fwd_ws.argtypes = [vp] * 5 + [sz] + [ci] * 5 + [vp]
        lib.based_fwd_ws.restype = ci
        lib.based_fwd_strerror.argtypes = [ci]
        lib.based_fwd_strerror.restype = ctypes.c_char_p
        lib.tile_mfma_calibrate_out_floats.argtypes = []
        lib.tile_mfma_calibrate_out_floats.restype = sz
        lib.tile_mfma_calibrate.argtypes = [vp, sz, ci, ci, ctypes.POINTER(ctypes.c_double), vp]
        lib.tile_mfma_calibrate.restype = ci
        _lib = lib
        return lib


def strerror(code: int) -> str:
    return load_library().attn_fwd_strerror(int(code)).decode()


def _current_stream_handle(device) -> int:
    import torch
    return int(torch.cuda.current_stream(device).cuda_stream)


def _stream_handle(stream, device) -> int:
    if stream is None:
        return _current_stream_handle(device)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check_bf16(name, t):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must have shape [B, H, N, D]")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
             stream=None, kernel: str = "auto"):
    """Fused softmax attention forward on the GPU.

    q, k, v: contiguous bfloat16 CUDA tensors of shape [B, H, N, D], D in {64, 128}.
    Returns (O bfloat16 [B, H, N, D], lse float32 [B, H, N]); ``out``/``lse`` may be
    given to write in place. ``scale`` defaults to 1/sqrt(D). The call is asynchronous
    on ``stream`` (a torch.cuda.Stream or raw handle; default: torch's current stream).
    ``kernel`` "auto" calls attn_fwd; "pingpong" or "fourwave" calls attn_fwd_ex with
    that kernel forced (tests and tuning; both give identical results).
    """
    import torch

    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    B, H, N, D = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, N] on q's device")
    if kernel not in FWD_KERNELS:
        raise ValueError(f"kernel must be one of {sorted(FWD_KERNELS)}")
    handle = _stream_handle(stream, q.device)
    lib = load_library()
    if kernel == "auto":
        code = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, N, D, int(bool(causal)), float(scale), handle)
    else:
        code = lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, N, D, int(bool(causal)), float(scale),
                               FWD_KERNELS[kernel], handle)
    if code != ATTN_FWD_OK:
        msg = lib.attn_fwd_strerror(code).decode()
        if code in (ATTN_FWD_EINVAL, ATTN_FWD_EUNSUPPORTED, ATTN_FWD_EALIGN):
            raise ValueError(f"attn_fwd rejected its arguments (code {code}): {msg}")
        raise AttnFwdError(code, msg)
    return out, lse


class AttnBwdError(RuntimeError):
    """A nonzero return code from attn_bwd."""

    def __init__(self, code: int, message: str):
        super().__init__(f"attn_bwd failed with code {code}: {message}")
        self.code = code


def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(int(B), int(H), int(N)))


def attn_bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Attention backward on the GPU: returns (dQ, dK, dV), bfloat16 [B, H, N, D].

    q, k, v, o, dout: contiguous bfloat16 CUDA tensors [B, H, N, D] (o and lse from
    attn_fwd with the same causal and scale); lse: float32 [B, H, N]. dq/dk/dv may be
    given to write in place; ``workspace`` (a uint8 CUDA tensor of at least
    bwd_workspace_bytes(B, H, N) bytes, 256-byte aligned) is allocated when not given.
    Asynchronous on ``stream`` (default: torch's current stream).
    """
    import torch

    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_bf16(name, t)
    if not (q.shape == k.shape == v.shape == o.shape == dout.shape):
        raise ValueError("q, k, v, o, dout must have one shape")
    if len({t.device for t in (q, k, v, o, dout)}) != 1:
        raise ValueError("all tensors must be on the same device")
    B, H, N, D = (int(x) for x in q.shape)
    if (not isinstance(lse, torch.Tensor) or tuple(lse.shape) != (B, H, N)
            or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, N] on q's device")
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check_bf16(name, t)
            if t.shape != q.shape or t.device != q.device:
                raise ValueError(f"{name} must be shaped like q on q's device")
        outs.append(t)
    lib = load_library()
    need = int(lib.attn_bwd_workspace_bytes(B, H, N))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif (workspace.dtype != torch.uint8 or workspace.device != q.device
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    handle = _stream_handle(stream, q.device)
    code = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                        lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                        workspace.data_ptr(), workspace.numel(), B, H, N, D, int(bool(causal)),
                        float(scale), handle)
    if code != ATTN_FWD_OK:
        msg = lib.attn_bwd_strerror(code).decode()
        if code in (ATTN_FWD_EINVAL, ATTN_FWD_EUNSUPPORTED, ATTN_FWD_EALIGN, ATTN_BWD_EWORKSPACE):
            raise ValueError(f"attn_bwd rejected its arguments (code {code}): {msg}")
        raise AttnBwdError(code, msg)
    return tuple(outs)


class AttnDecodeError(RuntimeError):
    """A nonzero return code from attn_decode."""

    def __init__(self, code: int, message: str):
        super().__init__(f"attn_decode failed with code {code}: {message}")
        self.code = code


def decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, D: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(D)))


def attn_decode(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
                workspace=None, stream=None):
    """Decode-shaped attention on the GPU: q [B, H, Nq, D] (Nq <= 32) against k, v
    [B, H, Nk, D], all contiguous bfloat16 CUDA tensors. Causal queries are the last Nq
    positions. Returns (O bfloat16 [B, H, Nq, D], lse float32 [B, H, Nq]); the workspace
    (uint8 CUDA tensor, 256-byte aligned) is allocated when not given."""
    import torch

    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"shapes do not match: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if len({t.device for t in (q, k, v)}) != 1:
        raise ValueError("q, k, v must be on the same device")
    B, H, Nq, D = (int(x) for x in q.shape)
    Nk = int(k.shape[2])
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must be shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, Nq] on q's device")
    lib = load_library()
    need = int(lib.attn_decode_workspace_bytes(B, H, Nq, Nk, D))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif (workspace.dtype != torch.uint8 or workspace.device != q.device
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    handle = _stream_handle(stream, q.device)
    code = lib.attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           workspace.data_ptr(), workspace.numel(), B, H, Nq, Nk, D,
                           int(bool(causal)), float(scale), handle)
    if code != ATTN_FWD_OK:
        msg = lib.attn_decode_strerror(code).decode()
        if code in (ATTN_FWD_EINVAL, ATTN_FWD_EUNSUPPORTED, ATTN_FWD_EALIGN, ATTN_BWD_EWORKSPACE):
            raise ValueError(f"attn_decode rejected its arguments (code {code}): {msg}")
        raise AttnDecodeError(code, msg)
    return out, lse


def attn_decode_noalloc(q, k, v, causal: bool = False, scale: float | None = None, out=None,
                        lse=None, stream=None):
    """attn_decode without a workspace: the C entry point keeps the per-chunk partials in a
    fixed device array of its own (ATTN_DECODE_NOALLOC_MAX_WORKSPACE bytes per GPU), so the
    library allocates nothing. ``out`` and ``lse`` are allocated here with torch when not
    given. Calls that overlap in time on one GPU share that array and race."""
    import torch

    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"shapes do not match: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if len({t.device for t in (q, k, v)}) != 1:
        raise ValueError("q, k, v must be on the same device")
    B, H, Nq, D = (int(x) for x in q.shape)
    Nk = int(k.shape[2])
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out)
        if out.shape != q.shape or out.device != q.device:
            raise ValueError("out must be shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, Nq] on q's device")
    lib = load_library()
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        code = lib.attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), B, H, Nq, Nk, D, int(bool(causal)),
                                       float(scale), handle)
    if code != ATTN_FWD_OK:
        msg = lib.attn_decode_strerror(code).decode()
        if code in (ATTN_FWD_EINVAL, ATTN_FWD_EUNSUPPORTED, ATTN_FWD_EALIGN, ATTN_BWD_EWORKSPACE):
            raise ValueError(f"attn_decode_noalloc rejected its arguments (code {code}): {msg}")
        raise AttnDecodeError(code, msg)
    return out, lse


class GemmError(RuntimeError):
    """A nonzero return code from gemm_bf16_nt."""

    def __init__(self, code: int, message: str):
        super().__init__(f"gemm_bf16_nt failed with code {code}: {message}")
        self.code = code


def gemm_nt(a, b, out=None, stream=None):
    """C = A B^T on the GPU: a [M, K], b [N, K] contiguous bfloat16 CUDA tensors (K and N
    multiples of 8). Returns C bfloat16 [M, N] (``out`` to write in place)."""
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 2-D bfloat16 GPU tensor")
    if a.shape[1] != b.shape[1] or a.device != b.device:
        raise ValueError(f"a {tuple(a.shape)} and b {tuple(b.shape)} must share K and the device")
    M, K = (int(x) for x in a.shape)
    N = int(b.shape[0])
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    elif (tuple(out.shape) != (M, N) or out.dtype != torch.bfloat16 or not out.is_contiguous()
          or out.device != a.device):
        raise ValueError("out must be a contiguous bfloat16 [M, N] tensor on a's device")
    lib = load_library()
    code = lib.gemm_bf16_nt(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                            _stream_handle(stream, a.device))
    if code != ATTN_FWD_OK:
        msg = lib.gemm_strerror(code).decode()
        if code in (ATTN_FWD_EINVAL, ATTN_FWD_EALIGN):
            raise ValueError(f"gemm_bf16_nt rejected its arguments (code {code}): {msg}")
        raise GemmError(code, msg)
    return out


BASED_D = 16
BASED_DV = 64


class BasedFwdError(RuntimeError):
    """A nonzero return code from based_fwd."""

    def __init__(self, code: int, message: str):
        super().__init__(f"based_fwd failed with code {code}: {message}")
        self.code = code


def based_fwd_workspace_bytes(B: int, H: int, N: int) -> int:
    """Workspace for based_fwd to split each head's sequence on the current device (0: no
    split pays)."""
    return int(load_library().based_fwd_workspace_bytes(int(B), int(H), int(N)))


def based_fwd(q, k, v, out=None, workspace=None, split=True, stream=None):
    """Based linear attention (causal) on the GPU: q, k [B, H, N, 16] and v [B, H, N, 64],
    contiguous bfloat16 CUDA tensors on one device. Returns o bfloat16 [B, H, N, 64]
    (``out`` to write in place). When B*H leaves compute units idle and ``split`` is true,
    each head's sequence is split over several workgroups (based_fwd_ws); ``workspace`` (a
    uint8 CUDA tensor of at least based_fwd_workspace_bytes(B, H, N) bytes) is allocated
    when not given."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    if q.shape != k.shape or v.shape[:3] != q.shape[:3] or q.device != k.device or q.device != v.device:
        raise ValueError(f"q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}: expected q, k "
                         "[B,H,N,d] and v [B,H,N,dv] on one device")
    B, H, N, d = (int(x) for x in q.shape)
    dv = int(v.shape[3])
    if d != BASED_D or dv != BASED_DV:
        raise ValueError(f"based_fwd needs d = {BASED_D} and dv = {BASED_DV}, got {d} and {dv}")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=torch.bfloat16, device=q.device)
    elif (tuple(out.shape) != (B, H, N, dv) or out.dtype != torch.bfloat16 or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous bfloat16 [B, H, N, 64] tensor on q's device")
    lib = load_library()
    need = int(lib.based_fwd_workspace_bytes(B, H, N)) if split else 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif (workspace.dtype != torch.uint8 or workspace.device != q.device
              or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
        code = lib.based_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                workspace.data_ptr(), workspace.numel(), B, H, N, d, dv,
                                _stream_handle(stream, q.device))
    else:
        code = lib.based_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d, dv,
                             _stream_handle(stream, q.device))
    if code != ATTN_FWD_OK:
        msg = lib.based_fwd_strerror(code).decode()
        if code in (ATTN_FWD_EINVAL, ATTN_FWD_EUNSUPPORTED, ATTN_FWD_EALIGN):
            raise ValueError(f"based_fwd rejected its arguments (code {code}): {msg}")
        raise BasedFwdError(code, msg)
    return out


def mfma_calibrate(iterations: int, random_operands: bool, out=None, stream=None) -> float:
    """Enqueue the sustained matrix-core probe (include/tile_calibrate.h) on the current
    CUDA device and return the floating-point operations it performs. ``out`` (float32,
    at least tile_mfma_calibrate_out_floats() elements) is allocated when not given; time
    the call with events on ``stream`` (default: torch's current stream)."""
    import torch

    lib = load_library()
    need = int(lib.tile_mfma_calibrate_out_floats())
    if need == 0:
        raise RuntimeError("tile_mfma_calibrate_out_floats: device query failed")
    dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty(need, dtype=torch.float32, device=dev)
    flops = ctypes.c_double(0.0)
    code = lib.tile_mfma_calibrate(out.data_ptr(), out.numel(), int(iterations),
                                   int(bool(random_operands)), ctypes.byref(flops),
                                   _stream_handle(stream, dev))
    if code != 0:
        raise RuntimeError(f"tile_mfma_calibrate failed with code {code}")
    return flops.value
