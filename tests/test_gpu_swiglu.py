"""GPU parity of the SwiGLU TP block share: AG GEMM with the silu(u)*v
epilogue, then the RS GEMM, against the oracle."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def run_block(case, inp, flags=0):
    xs = [dev(x) for x in inp["x_shards"]]
    w13, w2 = dev(inp["w13"]), dev(inp["w2"])
    h = bf16_empty(case.M, case.F)
    tp.stage_ag(xs, w13, None, h, M=case.M, N=2 * case.F, K=case.D, rank=case.rank, b_layout=tp.B_KN,
                epilogue=tp.EPI_SWIGLU, alpha=1.0, beta=0.0, flags=flags)
    out = bf16_empty(case.M, case.D)
    tp.stage_rs(h, w2, None, out, M=case.M, N=case.D, K=case.F, P=case.P, rank=case.rank,
                b_layout=tp.B_KN, flags=flags)
    torch.cuda.synchronize()
    return host_f64(h), host_f64(out)


@pytest.mark.parametrize("case", W.SMALL_SWIGLU, ids=lambda c: c.name)
def test_swiglu_block_parity(case):
    inp = W.swiglu_inputs(case)
    h_ref = oracle.swiglu_hidden(inp["x_shards"], inp["w13"])
    out_ref = oracle.swiglu_block(inp["x_shards"], inp["w13"], inp["w2"])
    res = []
    for name, flags in {"default": 0, "graph": tp.FORCE_GRAPH, "unstaged": tp.UNSTAGED, "eager": tp.NO_GRAPH}.items():
        say(f"swiglu: {case.name} mode={name}")
        h, out = run_block(case, inp, flags)
        assert_parity(h, h_ref, f"h/{name}")
        for blk in range(case.P):
            rows = slice(blk * case.S, (blk + 1) * case.S)
            assert_parity(out[rows], out_ref[rows], f"out/{name}/block{blk}")
        res.append(out)
    assert all(np.array_equal(r, res[0]) for r in res)
