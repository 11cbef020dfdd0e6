"""GPU check of the sustained matrix-core probe (include/tile_calibrate.h): it runs, reports
the flop count of its grid, and its products are what the operands fix (zero operands give
exactly zero; random operands in [-1, 1) give finite sums)."""
from __future__ import annotations

import pytest
import torch

from softmax_attention_fwd_amd import load_library, mfma_calibrate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def test_probe_runs_and_counts_flops():
    n = int(load_library().tile_mfma_calibrate_out_floats())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert n == 2 * cus * 256
    out = torch.full((n,), float("nan"), device="cuda")
    flops = mfma_calibrate(3, False, out=out)
    torch.cuda.synchronize()
    # 2 workgroups per CU, 4 waves each, 32 MFMAs of 32x32x16 per iteration
    assert flops == 2.0 * 32 * 32 * 16 * 32 * 3 * (2 * cus) * 4
    assert torch.equal(out, torch.zeros_like(out))
    mfma_calibrate(3, True, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and out.abs().max() > 0


def test_probe_rejects_short_output():
    lib = load_library()
    import ctypes
    out = torch.empty(16, device="cuda")
    flops = ctypes.c_double(0.0)
    assert lib.tile_mfma_calibrate(out.data_ptr(), 16, 3, 1, ctypes.byref(flops), None) == -1
