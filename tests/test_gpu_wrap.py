"""Staged runs that pass the last slice (or block) and go on from slice 0: with
slices of a multiple of 256 rows they run as one launch whose tiles past the
wrap write (and read A, in place) P * m rows earlier. Every rank of each
case, explicit stage groups (the one-launch carried form never applies),
parity with the oracle and bitwise identity with the unstaged call. The
in-place forms read the slices back to back from slice 0 (one launch) or
from separate allocations (one launch per stretch)."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

AG_CASES = [
    W.AgCase("wrap_ag_bf16_p4", M=4 * 256, N=520, K=256, P=4, dist="u11", alpha=0.5, beta=1.0),
    W.AgCase("wrap_ag_e4m3_p4", M=4 * 256, N=264, K=512, P=4, dtype="e4m3", dist="n05", c_dist="n01"),
    W.AgCase("wrap_ag_bf16_p4_kn_swiglu", M=4 * 256, N=2 * 264, K=256, P=4, b_layout="kn", dist="n05",
             beta=0.0, swiglu=True),
    W.AgCase("wrap_ag_bf16_p8", M=8 * 256, N=328, K=128, P=8, dist="u11", beta=-1.0),
]


def ag_call(case, slices, b, c, rank, flags, groups):
    nout = case.N // 2 if case.swiglu else case.N
    d = bf16_empty(case.M, nout)
    tp.stage_ag(slices, b, c, d, M=case.M, N=case.N, K=case.K, rank=rank,
                dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
                b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK,
                epilogue=tp.EPI_SWIGLU if case.swiglu else tp.EPI_ALPHA_BETA,
                alpha=case.alpha, beta=case.beta, flags=flags, groups=groups)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("case", AG_CASES, ids=lambda c: c.name)
def test_ag_wrapping_runs(case):
    inp = W.ag_inputs(case)
    apart = [dev(s) for s in inp["a_slices"]]
    whole = dev(np.concatenate(inp["a_slices"], axis=0))
    joined = [whole[s * case.m:(s + 1) * case.m] for s in range(case.P)]
    b = dev(inp["b"])
    c = dev(inp["c"]) if inp["c"] is not None else None
    for r in range(case.P):
        ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, r, case.dtype,
                             case.b_layout, swiglu=case.swiglu)
        say(f"wrap ag: {case.name} rank {r} unstaged")
        base = ag_call(case, apart, b, c, r, tp.UNSTAGED, 0)
        assert_parity(host_f64(base), ref, f"{case.name}/rank {r}/unstaged")
        base = base.cpu()
        for groups in (1, 2, 3):
            for label, slices, flags in (("copied", apart, 0), ("eager", apart, tp.NO_GRAPH),
                                         ("graph", apart, tp.FORCE_GRAPH), ("serial", apart, tp.SERIAL_STAGES),
                                         ("in place joined", joined, tp.NO_COPY),
                                         ("in place apart", apart, tp.NO_COPY)):
                say(f"wrap ag: {case.name} rank {r} groups {groups} {label}")
                d = ag_call(case, slices, b, c, r, flags, groups)
                assert_parity(host_f64(d), ref, f"{case.name}/rank {r}/groups {groups}/{label}")
                assert torch.equal(d.cpu(), base), f"{case.name}/rank {r}/groups {groups}/{label}"


RS_CASES = [
    W.RsCase("wrap_rs_bf16_p4", M=4 * 256, N=520, K=256, P=4, std=0.5),
    W.RsCase("wrap_rs_bf16_p8_kn", M=8 * 256, N=264, K=192, P=8, b_layout="kn", std=0.5, alpha=0.75),
]


@pytest.mark.parametrize("case", RS_CASES, ids=lambda c: c.name)
def test_rs_wrapping_runs(case):
    base_inp = W.rs_inputs(case)
    a, b = dev(base_inp["a"]), dev(base_inp["b"])
    m = case.m
    for r in range(case.P):
        # the generator's partials, moved round so that the slot of rank r
        # is the empty one
        inc_host = [base_inp["incoming"][(i - r + case.rank) % case.P] for i in range(case.P)]
        assert inc_host[r] is None and sum(x is None for x in inc_host) == 1
        inc = [dev(x) if x is not None else None for x in inc_host]
        ref = oracle.gemm_rs(base_inp["a"], base_inp["b"], inc_host, case.alpha, r, case.P, case.b_layout)
        outs = []
        for flags, groups in ((tp.UNSTAGED, 0), (0, 0), (tp.NO_GRAPH, 1), (tp.FORCE_GRAPH, 2), (tp.NO_COPY, 3),
                              (tp.SERIAL_STAGES, 1)):
            say(f"wrap rs: {case.name} rank {r} flags {flags} groups {groups}")
            d = bf16_empty(case.M, case.N)
            tp.stage_rs(a, b, inc, d, M=case.M, N=case.N, K=case.K, P=case.P, rank=r,
                        b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK, alpha=case.alpha,
                        flags=flags, groups=groups)
            torch.cuda.synchronize()
            got = host_f64(d)
            for blk in range(case.P):
                rows = slice(blk * m, (blk + 1) * m)
                assert_parity(got[rows], ref[rows], f"{case.name}/rank {r}/flags {flags}/block {blk}")
            outs.append(d.cpu())
        assert all(torch.equal(o, outs[0]) for o in outs), f"{case.name}/rank {r}"


# Rotating B: a run of delivered B column slices that passes slice P-1 is one
# launch whose tiles past the wrap write D's and C's columns P * n earlier
# (slices of a multiple of 256 columns).
ROTB_CASES = [
    W.AgCase("wrap_rotb_bf16_p4", M=4 * 64, N=4 * 256, K=256, P=4, dist="u11", alpha=0.5, beta=1.0),
    W.AgCase("wrap_rotb_e4m3_p4", M=4 * 128, N=4 * 256, K=512, P=4, dtype="e4m3", dist="n05", c_dist="n01"),
    W.AgCase("wrap_rotb_bf16_p4_kn", M=4 * 64, N=4 * 256, K=192, P=4, b_layout="kn", dist="u11", beta=-1.0),
]


@pytest.mark.parametrize("case", ROTB_CASES, ids=lambda c: c.name)
def test_ag_rotb_wrapping_runs(case):
    inp = W.ag_rotb_inputs(case)
    a = dev(inp["a"])
    bs = [dev(x) for x in inp["b_slices"]]
    c = dev(inp["c"]) if inp["c"] is not None else None

    def call(rank, flags, groups):
        d = bf16_empty(case.M, case.N)
        tp.stage_ag(a, bs, c, d, M=case.M, N=case.N, K=case.K, rank=rank,
                    dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
                    b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK,
                    alpha=case.alpha, beta=case.beta, flags=flags, groups=groups, schedule=tp.ROTATE_B)
        torch.cuda.synchronize()
        return d

    for r in range(case.P):
        ref = oracle.gemm_ag_rotb(inp["a"], inp["b_slices"], inp["c"], case.alpha, case.beta, r, case.dtype,
                                  case.b_layout)
        say(f"wrap rotb: {case.name} rank {r} unstaged")
        base = call(r, tp.UNSTAGED, 0)
        assert_parity(host_f64(base), ref, f"{case.name}/rank {r}/unstaged")
        base = base.cpu()
        for groups in (0, 1, 2, 3):
            for label, flags in (("default", 0), ("eager", tp.NO_GRAPH), ("graph", tp.FORCE_GRAPH),
                                 ("serial", tp.SERIAL_STAGES), ("in place", tp.NO_COPY)):
                say(f"wrap rotb: {case.name} rank {r} groups {groups} {label}")
                d = call(r, flags, groups)
                assert_parity(host_f64(d), ref, f"{case.name}/rank {r}/groups {groups}/{label}")
                assert torch.equal(d.cpu(), base), f"{case.name}/rank {r}/groups {groups}/{label}"


def random_plans(seed, count):
    """Seeded stage plans: slice heights that take the one-launch wrap (256,
    512) and the per-stretch launches (128, 320), any rank and grouping."""
    rng = np.random.default_rng(seed)
    plans = []
    for i in range(count):
        P = int(rng.choice([2, 3, 4, 5, 8]))
        m = int(rng.choice([128, 256, 320, 512]))
        dtype = str(rng.choice(["bf16", "e4m3"]))
        layout = "nk" if dtype == "e4m3" else str(rng.choice(["nk", "kn"]))
        K = int(rng.choice([256, 384])) * (2 if dtype == "e4m3" else 1)
        N = int(rng.choice([264, 512]))
        rank = int(rng.integers(0, P))
        groups = int(rng.integers(1, P)) if P > 1 else 1
        plans.append((f"plan{seed}_{i}", P, m, dtype, layout, K, N, rank, groups))
    return plans


@pytest.mark.parametrize("plan", random_plans(7, 16), ids=lambda p: p[0])
def test_ag_random_stage_plans(plan):
    name, P, m, dtype, layout, K, N, rank, groups = plan
    case = W.AgCase(name, M=P * m, N=N, K=K, P=P, rank=rank, dtype=dtype, b_layout=layout,
                    dist="n05" if dtype == "e4m3" else "u11", c_dist="n01" if dtype == "e4m3" else "u11",
                    alpha=0.75, beta=1.0)
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, rank, dtype, layout)
    apart = [dev(s) for s in inp["a_slices"]]
    whole = dev(np.concatenate(inp["a_slices"], axis=0))
    joined = [whole[s * m:(s + 1) * m] for s in range(P)]
    b, c = dev(inp["b"]), dev(inp["c"])
    say(f"random plan: {name} P={P} m={m} {dtype}/{layout} K={K} N={N} rank={rank} groups={groups} unstaged")
    base = ag_call(case, apart, b, c, rank, tp.UNSTAGED, 0)
    assert_parity(host_f64(base), ref, f"{name}/unstaged")
    base = base.cpu()
    for label, slices, flags in (("copied", apart, 0), ("graph", apart, tp.FORCE_GRAPH),
                                 ("in place joined", joined, tp.NO_COPY), ("serial", apart, tp.SERIAL_STAGES)):
        say(f"random plan: {name} {label}")
        d = ag_call(case, slices, b, c, rank, flags, groups)
        assert_parity(host_f64(d), ref, f"{name}/{label}")
        assert torch.equal(d.cpu(), base), f"{name}/{label}"


@pytest.mark.parametrize("plan", random_plans(11, 10), ids=lambda p: p[0])
def test_rs_random_stage_plans(plan):
    name, P, m, _, layout, K, N, rank, groups = plan
    case = W.RsCase(name, M=P * m, N=N, K=K, P=P, rank=rank, b_layout=layout, std=0.5, alpha=1.25)
    inp = W.rs_inputs(case)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], case.alpha, rank, P, layout)
    outs = []
    for flags, g in ((tp.UNSTAGED, 0), (0, 0), (tp.FORCE_GRAPH, groups), (tp.NO_COPY, groups),
                     (tp.SERIAL_STAGES, groups)):
        say(f"random plan: {name} P={P} m={m} {layout} K={K} N={N} rank={rank} flags={flags} groups={g}")
        d = bf16_empty(case.M, case.N)
        tp.stage_rs(a, b, inc, d, M=case.M, N=case.N, K=case.K, P=P, rank=rank,
                    b_layout=tp.B_KN if layout == "kn" else tp.B_NK, alpha=case.alpha, flags=flags, groups=g)
        torch.cuda.synchronize()
        got = host_f64(d)
        for blk in range(P):
            rows = slice(blk * m, (blk + 1) * m)
            assert_parity(got[rows], ref[rows], f"{name}/flags {flags}/block {blk}")
        outs.append(d.cpu())
    assert all(torch.equal(o, outs[0]) for o in outs), name
