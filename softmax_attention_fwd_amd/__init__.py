"""MI355X-native fused softmax attention (gfx950 HIP kernels behind a C ABI).

``attn_fwd``, ``attn_bwd``, ``attn_decode``, ``gemm_nt`` and ``based_fwd`` are thin Python bindings over
``libattn_fwd.so``; the
library is loaded on first use and its absence is an error (there is no fallback path).
"""
from .binding import (AttnBwdError, AttnDecodeError, AttnFwdError, BasedFwdError, GemmError,
                      attn_bwd, attn_decode, attn_decode_noalloc, attn_fwd, based_fwd, bwd_workspace_bytes,
                      decode_workspace_bytes, gemm_nt, library_path, load_library, mfma_calibrate)

__all__ = ["attn_fwd", "attn_bwd", "attn_decode", "attn_decode_noalloc", "gemm_nt", "based_fwd", "bwd_workspace_bytes",
           "decode_workspace_bytes", "library_path", "load_library", "AttnFwdError", "AttnBwdError",
           "AttnDecodeError", "GemmError", "BasedFwdError", "mfma_calibrate"]
