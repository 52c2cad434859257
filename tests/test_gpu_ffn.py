"""GPU parity of the per-token-slot FFN against the oracle."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def run_ffn(case, inp, flags):
    t = {k: dev(v) for k, v in inp.items()}
    y = bf16_empty(case.PB, case.L, case.D)
    tp.ffn_slot_forward(t["x"], t["w1"], t["b1"], t["wout"], t["bout"], t["gx"], t["bx"], t["gg"], t["bg"],
                        y, PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps, flags=flags)
    torch.cuda.synchronize()
    return host_f64(y)


FFN_CASES = W.SMALL_FFN + [W.FfnCase("ffn_mid_ragged", B=9, T=32, D=264, k=3, P=4, rank=2, big_bias=True),
                           W.FfnCase("ffn_dma_ragged", B=5, T=16, D=192, k=2, P=4, rank=1, affine=True),
                           # 8 slots of a second GEMM with 2 x 2 tiles of 256 x 256 each: the batched launch
                           # gives each XCD whole slots, so every tile must pair with its own slot
                           W.FfnCase("ffn_eight_slots_many_tiles", B=64, T=64, D=512, k=2, P=8, affine=True)]


@pytest.mark.parametrize("case", FFN_CASES, ids=lambda c: c.name)
def test_ffn_parity(case):
    inp = W.ffn_inputs(case)
    ref = oracle.ffn_slot_forward(inp, case.eps)
    outs = []
    for name, flags in {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "serial": tp.SERIAL_STAGES}.items():
        say(f"ffn: {case.name} mode={name}")
        got = run_ffn(case, inp, flags)
        assert_parity(got, ref, f"{case.name}/{name}")
        outs.append(got)
    assert all(np.array_equal(o, outs[0]) for o in outs)
