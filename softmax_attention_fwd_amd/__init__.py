"""MI355X-native fused softmax attention forward (gfx950 HIP kernels behind a C ABI).

``attn_fwd`` is the thin Python binding over ``libattn_fwd.so``; the library is loaded
on first use and its absence is an error (there is no fallback path).
"""
from .binding import attn_fwd, library_path, load_library, AttnFwdError

__all__ = ["attn_fwd", "library_path", "load_library", "AttnFwdError"]
