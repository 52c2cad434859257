"""GPU parity of the staged GEMM + reduce-scatter share against the oracle."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

MODES = {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "unstaged": tp.UNSTAGED,
         "no_copy": tp.NO_COPY, "serial": tp.SERIAL_STAGES, "shader": tp.COPY_SHADER | tp.NO_GRAPH,
         "kernel": tp.COPY_KERNEL}


def run_rs(case, inp, flags, incoming=True):
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]] if incoming else None
    d = bf16_empty(case.M, case.N)
    tp.stage_rs(a, b, inc, d, M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank,
                b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK, alpha=case.alpha, flags=flags)
    torch.cuda.synchronize()
    return host_f64(d)


@pytest.mark.parametrize("case", W.SMALL_RS, ids=lambda c: c.name)
def test_rs_parity_all_modes(case):
    inp = W.rs_inputs(case)
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], case.alpha, case.rank, case.P, case.b_layout)
    m, r = case.m, case.rank
    outs = {}
    for name, flags in MODES.items():
        say(f"rs: {case.name} mode={name}")
        got = run_rs(case, inp, flags)
        for blk in range(case.P):           # tolerance per block
            rows = slice(blk * m, (blk + 1) * m)
            assert_parity(got[rows], ref[rows], f"{case.name}/{name}/block{blk}")
        outs[name] = got
    for name in MODES:
        assert np.array_equal(outs[name], outs["default"]), name
    # the own block without incoming partials is the plain partial product
    say(f"rs: {case.name} own block without incoming")
    got0 = run_rs(case, inp, 0, incoming=False)
    ref0 = oracle.gemm_rs(inp["a"], inp["b"], None, case.alpha, r, case.P, case.b_layout)
    assert_parity(got0, ref0, "no incoming")
    # own partial recovered from the reduced block: out_r - sum(incoming) ~ E_r,
    # at a tolerance scaled to E_r itself (the incoming sum dominates out_r)
    rows = slice(r * m, (r + 1) * m)
    inc_sum = sum(oracle.decode_bf16(x) for x in inp["incoming"] if x is not None)
    own = outs["default"][rows] - inc_sum
    e_r = ref0[rows]
    rms_e = np.sqrt(np.mean(e_r ** 2))
    ulp_out = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref[rows]), 1e-30))) - 7)
    assert np.all(np.abs(own - e_r) <= 0.02 * rms_e + ulp_out), "own partial mis-scaled or missing"


@pytest.mark.parametrize("contiguous", [False, True])
def test_rs_groups_are_bitwise_identical(contiguous):
    case = W.RsCase("rs_groups", M=8 * 64, N=264, K=192, P=8, rank=6, std=0.5)
    inp = W.rs_inputs(case)
    a, b = dev(inp["a"]), dev(inp["b"])
    if contiguous:
        peers = [j for j in range(case.P) if j != case.rank]
        whole = dev(np.concatenate([inp["incoming"][j] for j in peers], axis=0))
        inc = [None] * case.P
        for i, j in enumerate(peers):
            inc[j] = whole[i * case.m:(i + 1) * case.m]
    else:
        inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], 1.0, case.rank, case.P)
    outs = []
    for groups in (0, 1, 3, 7):
        for flags in (0, tp.FORCE_GRAPH, tp.NO_GRAPH, tp.NO_COPY):
            say(f"rs groups: contiguous={contiguous} groups={groups} flags={flags}")
            d = bf16_empty(case.M, case.N)
            tp.stage_rs(a, b, inc, d, M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank, flags=flags,
                        groups=groups)
            torch.cuda.synchronize()
            outs.append(d.cpu())
    got = host_f64(d)
    for blk in range(case.P):
        rows = slice(blk * case.m, (blk + 1) * case.m)
        assert_parity(got[rows], ref[rows], f"block {blk}")
    assert all(torch.equal(o, outs[0]) for o in outs)
