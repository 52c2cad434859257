"""GPU parity of the column-dual schedules against the oracle, through the C
ABI: the all-gather with rotating B (TPG_ROTATE_B) and the reduce-scatter
with tiled B (TPG_TILE_B). Every issue mode must give the same bits."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

AG_MODES = {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "unstaged": tp.UNSTAGED,
            "no_copy": tp.NO_COPY, "serial": tp.SERIAL_STAGES, "sdma": tp.COPY_SDMA, "shader": tp.COPY_SHADER}
RS_MODES = {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "unstaged": tp.UNSTAGED,
            "no_copy": tp.NO_COPY, "serial": tp.SERIAL_STAGES, "shader": tp.COPY_SHADER, "kernel": tp.COPY_KERNEL}


def run_ag_rotb(case, inp, flags, groups=0, workspace=None):
    a = dev(inp["a"])
    bs = [dev(x) for x in inp["b_slices"]]
    c = dev(inp["c"]) if inp["c"] is not None else None
    d = bf16_empty(case.M, case.N)
    tp.stage_ag(a, bs, c, d, M=case.M, N=case.N, K=case.K, rank=case.rank,
                dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
                b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK,
                alpha=case.alpha, beta=case.beta, flags=flags, groups=groups, schedule=tp.ROTATE_B,
                workspace=workspace)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("case", W.SMALL_AG_ROTB, ids=lambda c: c.name)
def test_ag_rotb_parity_all_modes(case):
    inp = W.ag_rotb_inputs(case)
    ref = oracle.gemm_ag_rotb(inp["a"], inp["b_slices"], inp["c"], case.alpha, case.beta, case.rank,
                              case.dtype, case.b_layout)
    outs = {}
    for name, flags in AG_MODES.items():
        if name == "no_copy" and case.b_layout == "kn":
            flags = tp.NO_COPY          # staged in place (unstaged in place needs NK)
        say(f"ag rotb: {case.name} mode={name}")
        d = run_ag_rotb(case, inp, flags)
        assert_parity(host_f64(d), ref, f"{case.name}/{name}")
        outs[name] = d.cpu()
    for groups in (1, 2, case.P - 1):
        say(f"ag rotb: {case.name} groups={groups}")
        outs[f"g{groups}"] = run_ag_rotb(case, inp, 0, groups).cpu()
    for name, o in outs.items():
        assert torch.equal(o, outs["default"]), name


def run_rs_tileb(case, inp, flags, groups=0, workspace=None):
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    d = bf16_empty(case.M, case.N)
    tp.stage_rs(a, b, inc, d, M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank,
                b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK, alpha=case.alpha, flags=flags,
                groups=groups, schedule=tp.TILE_B, workspace=workspace)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("case", W.SMALL_RS_TILEB, ids=lambda c: c.name)
def test_rs_tileb_parity_all_modes(case):
    inp = W.rs_tileb_inputs(case)
    ref = oracle.gemm_rs_tileb(inp["a"], inp["b"], inp["incoming"], case.alpha, case.rank, case.P,
                               case.b_layout)
    outs = {}
    for name, flags in RS_MODES.items():
        say(f"rs tileb: {case.name} mode={name}")
        d = run_rs_tileb(case, inp, flags)
        got = host_f64(d)
        assert_parity(got, ref, f"{case.name}/{name}")
        outs[name] = d.cpu()
    for groups in (1, 3, case.P - 1):
        say(f"rs tileb: {case.name} groups={groups}")
        outs[f"g{groups}"] = run_rs_tileb(case, inp, 0, groups).cpu()
    for name, o in outs.items():
        assert torch.equal(o, outs["default"]), name
    # the emitted column blocks are the plain partial: the incoming partials
    # touch the own block only
    n = case.N // case.P
    plain = oracle.gemm_rs_tileb(inp["a"], inp["b"], None, case.alpha, case.rank, case.P, case.b_layout)
    got = host_f64(outs["default"])
    for blk in range(case.P):
        if blk != case.rank:
            cols = slice(blk * n, (blk + 1) * n)
            assert_parity(got[:, cols], plain[:, cols], f"emitted block {blk}")
    # own column block minus the incoming partials ~ alpha * E_rank, at a
    # tolerance scaled to that partial (the incoming sum dominates the block)
    cols = slice(case.rank * n, (case.rank + 1) * n)
    inc_sum = sum(oracle.decode_bf16(x) for x in inp["incoming"] if x is not None)
    own = got[:, cols] - inc_sum
    e_r = plain[:, cols]
    rms_e = np.sqrt(np.mean(e_r ** 2))
    ulp_out = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref[:, cols]), 1e-30))) - 7)
    assert np.all(np.abs(own - e_r) <= 0.02 * rms_e + ulp_out), "own partial mis-scaled or missing"


def test_column_duals_with_held_deliveries():
    """Deliveries held back behind a host sleep, receive slots poisoned with
    NaN: the gated stages still see their own slices."""
    hold = tp.DEBUG_HOLD_DELIVERIES
    case = W.SMALL_AG_ROTB[1]
    inp = W.ag_rotb_inputs(case)
    ref = oracle.gemm_ag_rotb(inp["a"], inp["b_slices"], inp["c"], case.alpha, case.beta, case.rank,
                              case.dtype, case.b_layout)
    for flags, groups in [(hold, 1), (hold, 3), (hold | tp.UNSTAGED, 0)]:
        say(f"gates rotb: flags={flags} groups={groups}")
        ws = torch.full((64 << 20,), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint8)
        d = run_ag_rotb(case, inp, flags, groups, workspace=ws)
        assert_parity(host_f64(d), ref, f"rotb hold {flags}/{groups}")
    rcase = W.SMALL_RS_TILEB[1]
    rinp = W.rs_tileb_inputs(rcase)
    rref = oracle.gemm_rs_tileb(rinp["a"], rinp["b"], rinp["incoming"], 1.0, rcase.rank, rcase.P, rcase.b_layout)
    for flags, groups in [(hold, 1), (hold | tp.COPY_SHADER, 3), (hold | tp.UNSTAGED, 0)]:
        say(f"gates tileb: flags={flags} groups={groups}")
        ws = torch.full((64 << 20,), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint8)
        d = run_rs_tileb(rcase, rinp, flags, groups, workspace=ws)
        got = host_f64(d)
        assert not np.isnan(got).any()
        assert_parity(got, rref, f"tileb hold {flags}/{groups}")
