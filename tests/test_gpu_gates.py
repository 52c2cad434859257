"""Ordering forced from the host: every delivery is held back behind a 20 ms
host callback while the stage runs that read it are already queued, and the
receive slots start out as NaN. The output must still match the oracle, so
each gated stage waited for its own slices (and never read a slot early)."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

HOLD = tp.DEBUG_HOLD_DELIVERIES


def poisoned(nbytes, elem_bytes):
    """A workspace whose every element is a NaN of the operand type."""
    if elem_bytes == 2:
        return torch.full((max(nbytes, 2) // 2,), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint8)
    return torch.full((max(nbytes, 1),), 0x7F, dtype=torch.uint8, device="cuda")   # e4m3 NaN


AG_CASES = [W.AgCase("gate_ag_bf16", M=8 * 96, N=264, K=256, P=8, rank=3, dist="u11"),
            W.AgCase("gate_ag_e4m3", M=4 * 128, N=200, K=512, P=4, rank=1, dtype="e4m3", dist="n05",
                     c_dist="n01")]


@pytest.mark.parametrize("case", AG_CASES, ids=lambda c: c.name)
def test_ag_gates_hold_with_delayed_deliveries(case):
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank, case.dtype)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    eb = 1 if case.dtype == "e4m3" else 2
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, dtype=tp.E4M3 if eb == 1 else tp.BF16,
              alpha=case.alpha, beta=case.beta)
    probe = bf16_empty(case.M, case.N)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, probe, flags=tp.UNSTAGED, **kw))
    for flags, groups in [(HOLD, 1), (HOLD, 3), (HOLD, case.P - 1), (HOLD | tp.COPY_SDMA, 3),
                          (HOLD | tp.UNSTAGED, 0)]:
        say(f"gates: {case.name} flags={flags} groups={groups}")
        ws = poisoned(need, eb)
        d = bf16_empty(case.M, case.N)
        tp.stage_ag(slices, b, c, d, flags=flags, groups=groups, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert_parity(host_f64(d), ref, f"{case.name}/flags={flags}/groups={groups}")


def test_rs_own_block_waits_for_delayed_partials():
    case = W.RsCase("gate_rs", M=8 * 96, N=264, K=192, P=8, rank=5, std=0.5)
    inp = W.rs_inputs(case)
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], 1.0, case.rank, case.P)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    kw = dict(M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank)
    probe = bf16_empty(case.M, case.N)
    need = tp.stage_rs_workspace_size(tp.rs_args(a, b, inc, probe, flags=tp.UNSTAGED, **kw))
    for flags, groups in [(HOLD, 1), (HOLD, 3), (HOLD | tp.COPY_SHADER, 3), (HOLD | tp.UNSTAGED, 0)]:
        say(f"gates: rs flags={flags} groups={groups}")
        ws = poisoned(need, 2)
        d = bf16_empty(case.M, case.N)
        tp.stage_rs(a, b, inc, d, flags=flags, groups=groups, workspace=ws, **kw)
        torch.cuda.synchronize()
        got = host_f64(d)
        assert not np.isnan(got).any()
        assert_parity(got, ref, f"rs/flags={flags}/groups={groups}")


# Latency-bound calls (under 1 GFLOP, library grouping) run on one stream and
# carry the deliveries inside the local stage's launch when its direct-to-LDS
# kernel runs (K * element size a multiple of 128 bytes), else copy first:
# both paths, each with a fresh poisoned workspace.
CARRY_CASES = [W.AgCase("gate_carry_bf16", M=8 * 96, N=264, K=256, P=8, rank=3, dist="u11"),
               W.AgCase("gate_carry_e4m3", M=4 * 64, N=136, K=384, P=4, rank=2, dtype="e4m3", dist="n05",
                        c_dist="n01"),
               W.AgCase("gate_copy_first_bf16", M=4 * 64, N=136, K=200, P=4, rank=1, dist="u11")]


@pytest.mark.parametrize("case", CARRY_CASES, ids=lambda c: c.name)
def test_latency_bound_ag_with_delayed_deliveries(case):
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank, case.dtype)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    eb = 1 if case.dtype == "e4m3" else 2
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, dtype=tp.E4M3 if eb == 1 else tp.BF16,
              alpha=case.alpha, beta=case.beta)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, bf16_empty(case.M, case.N), **kw))
    for flags in (HOLD, 0):
        say(f"gates latency-bound: {case.name} flags={flags} groups=0")
        ws = poisoned(need, eb)
        d = bf16_empty(case.M, case.N)
        tp.stage_ag(slices, b, c, d, flags=flags, groups=0, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert_parity(host_f64(d), ref, f"{case.name}/flags={flags}")


# Negative control: with TPG_DEBUG_NO_GATE the stage runs that read delivered
# data do not wait for their deliveries; held back 20 ms, those deliveries
# land long after the runs have read the NaN-poisoned slots. The gate tests
# above can therefore fail: the rows of every remote stage must be wrong here,
# while the local stage's rows (no delivery) stay right.
@pytest.mark.parametrize("groups", [1, 7])
def test_no_gate_negative_control_ag(groups):
    case = AG_CASES[0]
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank, case.dtype)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, alpha=case.alpha, beta=case.beta)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, bf16_empty(case.M, case.N), **kw))
    say(f"gates negative control: ag groups={groups}")
    ws = poisoned(need, 2)
    d = bf16_empty(case.M, case.N)
    tp.stage_ag(slices, b, c, d, flags=HOLD | tp.DEBUG_NO_GATE, groups=groups, workspace=ws, **kw)
    torch.cuda.synchronize()
    got = host_f64(d)
    m = case.m
    for s in range(case.P):
        rows = slice(s * m, (s + 1) * m)
        if s == case.rank:
            assert_parity(got[rows], ref[rows], "local stage")
        else:
            assert np.isnan(got[rows]).all(), f"stage of slice {s} read its slot after the delivery"


def test_no_gate_negative_control_rs():
    case = W.RsCase("gate_rs", M=8 * 96, N=264, K=192, P=8, rank=5, std=0.5)
    inp = W.rs_inputs(case)
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], 1.0, case.rank, case.P)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    kw = dict(M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank)
    need = tp.stage_rs_workspace_size(tp.rs_args(a, b, inc, bf16_empty(case.M, case.N), **kw))
    say("gates negative control: rs groups=1")
    ws = poisoned(need, 2)
    d = bf16_empty(case.M, case.N)
    tp.stage_rs(a, b, inc, d, flags=HOLD | tp.DEBUG_NO_GATE, groups=1, workspace=ws, **kw)
    torch.cuda.synchronize()
    got = host_f64(d)
    m, r = case.m, case.rank
    own = slice(r * m, (r + 1) * m)
    assert np.isnan(got[own]).all(), "own block read the partials after their delivery"
    emitted = np.ones(case.M, dtype=bool)
    emitted[own] = False
    assert_parity(got[emitted], ref[emitted], "emitted blocks")


def test_latency_bound_call_is_one_gated_launch():
    """A latency-bound staged call with library-chosen grouping runs as one
    GEMM launch that carries its deliveries and gates the delivered slices'
    tiles in-kernel (one launch record over all M rows); with a test flag
    that needs the deliveries on their own stream it keeps the two-launch
    schedule. Both match the oracle on a poisoned workspace."""
    case = W.AgCase("one_launch_bf16", M=8 * 128, N=264, K=256, P=8, rank=3, dist="u11")   # M/P % 128 == 0
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank, case.dtype)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, alpha=case.alpha, beta=case.beta)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, bf16_empty(case.M, case.N), **kw))
    # one gated launch; else the local stage, then the remote stages (one
    # launch per stretch of rows that does not wrap past slice P-1)
    for flags, launches in ((tp.PROFILE, 1), (tp.PROFILE | HOLD, 3)):
        say(f"latency-bound launch count: flags={flags}")
        ws = poisoned(need, 2)
        d = bf16_empty(case.M, case.N)
        tp.profile_read()
        tp.stage_ag(slices, b, c, d, flags=flags, groups=0, workspace=ws, **kw)
        torch.cuda.synchronize()
        recs = tp.profile_read()
        assert len(recs) == launches, recs
        assert sum(r[1] for r in recs) == pytest.approx(case.flop)
        assert_parity(host_f64(d), ref, f"flags={flags}")
