"""CPU oracle for the fused softmax attention passes and the plain GEMM (fp64).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path (the HIP
library and its Python binding) never imports, calls or links it, and the two share no
code. Modules:

  attention  the plain definition in numpy float64 (full tensors, selected rows, P matrix)
  brute      pure-Python loops with math.fsum, for tiny shapes
  online     the pages' tiled online-softmax recurrence in float64 (to pin the identity)
  backward   the gradients dQ, dK, dV of the forward definition, by the chain rule
  decode     few queries against a long key/value sequence (bottom-right causal mask)
  gemm       the plain matrix product C = A B^T
  based      Based linear attention (second-order Taylor feature map), causal

Every function here is pinned by ``tests/test_oracle.py``, ``tests/test_oracle_bwd.py``,
``tests/test_oracle_decode.py``, ``tests/test_oracle_gemm.py`` and
``tests/test_oracle_based.py``
against closed forms, invariants, a hand-derived worked example, brute force and finite
differences.
"""
from .attention import attention_fwd, attention_head, attention_probs, attention_rows
from .backward import attention_bwd, attention_bwd_head
from .decode import attention_decode
from .gemm import gemm_nt
from .based import based_linear_attention, based_recurrent
from .brute import attention_brute
from .online import attention_online

__all__ = [
    "attention_fwd",
    "attention_head",
    "attention_probs",
    "attention_rows",
    "attention_brute",
    "attention_online",
    "attention_bwd",
    "attention_bwd_head",
    "attention_decode",
    "gemm_nt",
    "based_linear_attention",
    "based_recurrent",
]
