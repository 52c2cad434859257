"""The register-only MFMA probe used by the bench to report the attainable
matrix-core rate: its flop count, tick records and rate must be plausible."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
from tests.devutil import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,flop_per_mfma,spec", [(tp.BF16, 2 * 32 * 32 * 16, 2500.0),
                                                      (tp.E4M3, 2 * 32 * 32 * 64, 5000.0)])
def test_mfma_probe(dtype, flop_per_mfma, spec):
    cus, clk_khz, wall_khz = tp.device_info()
    assert cus > 0 and clk_khz > 0 and wall_khz > 0
    blocks, iters = 2 * cus, 2000
    sink = torch.zeros(blocks * 8 * 2, dtype=torch.int64, device="cuda")
    say(f"probe: dtype={dtype} blocks={blocks} iters={iters}")
    tp.mfma_probe(dtype, iters, blocks, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    flop = tp.mfma_probe(dtype, iters, blocks, sink)
    e.record()
    torch.cuda.synchronize()
    assert flop == blocks * 8 * 4 * flop_per_mfma * iters
    ticks = sink.view(-1, 2).cpu().numpy()
    assert (ticks > 0).all()                              # every wave ran and recorded
    mhz = np.median(ticks[:, 0] / ticks[:, 1]) * wall_khz / 1e3
    assert 300 < mhz <= 1.05 * clk_khz / 1e3, mhz
    tf = flop / (s.elapsed_time(e) * 1e-3) / 1e12
    assert 0.2 * spec < tf <= 1.05 * spec, tf
