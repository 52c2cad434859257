"""GPU parity of the staged all-gather GEMM against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import gen, workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64, bf16_bits_of
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

MODES = {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "unstaged": tp.UNSTAGED,
         "no_copy": tp.NO_COPY, "serial": tp.SERIAL_STAGES | tp.NO_GRAPH, "sdma": tp.COPY_SDMA, "shader": tp.COPY_SHADER}


def run_ag(case, inp, flags, rank=None):
    slices = [dev(s) for s in inp["a_slices"]]
    if flags & tp.UNSTAGED and flags & tp.NO_COPY:
        raise ValueError("not used")
    b, c = dev(inp["b"]), dev(inp["c"])
    nout = case.N // 2 if case.swiglu else case.N
    d = bf16_empty(case.M, nout)
    tp.stage_ag(slices, b, c, d, M=case.M, N=case.N, K=case.K, rank=case.rank if rank is None else rank,
                dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
                b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK,
                epilogue=tp.EPI_SWIGLU if case.swiglu else tp.EPI_ALPHA_BETA,
                alpha=case.alpha, beta=case.beta, flags=flags)
    torch.cuda.synchronize()
    return d


def oracle_ag(case, inp):
    return oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank,
                          case.dtype, case.b_layout, swiglu=case.swiglu)


@pytest.mark.parametrize("case", W.SMALL_AG + [W.C1], ids=lambda c: c.name)
def test_ag_parity_all_modes(case):
    inp = W.ag_inputs(case)
    ref = oracle_ag(case, inp)
    outs = {}
    for name, flags in MODES.items():
        say(f"ag: {case.name} mode={name}")
        d = run_ag(case, inp, flags)
        assert_parity(host_f64(d), ref, f"{case.name}/{name}")
        outs[name] = d.cpu()
    # staging only partitions rows: every mode is bitwise identical
    for name in MODES:
        assert torch.equal(outs[name], outs["default"]), name


def test_ag_integer_inputs_are_bit_exact():
    """Inputs in {-1, 0, 1}: fp32 sums are exact, so D must equal the
    round-to-nearest-even of the exact result, bit for bit."""
    rng = np.random.default_rng(3)
    P, m, N, K = 4, 72, 136, 320
    slices = [gen.encode_bf16(rng.integers(-1, 2, (m, K))) for _ in range(P)]
    b = gen.encode_bf16(rng.integers(-1, 2, (N, K)))
    c = gen.encode_bf16(rng.integers(-3, 4, (P * m, N)) * 0.5)
    case = W.AgCase("int", M=P * m, N=N, K=K, P=P, rank=2, alpha=1.0, beta=1.0)
    say("ag: integer exactness")
    d = run_ag(case, dict(a_slices=slices, b=b, c=c), 0)
    ref = oracle.gemm_ag(slices, b, c, 1.0, 1.0, 2)
    assert np.array_equal(d.cpu().numpy(), bf16_bits_of(ref))
    # e4m3 with quarter-integers: still exact in fp32
    s8 = [gen.encode_e4m3(rng.integers(-4, 5, (m, K)) * 0.25) for _ in range(P)]
    b8 = gen.encode_e4m3(rng.integers(-4, 5, (N, K)) * 0.5)
    case8 = W.AgCase("int8", M=P * m, N=N, K=K, P=P, rank=1, dtype="e4m3", alpha=1.0, beta=0.0)
    d8 = run_ag(case8, dict(a_slices=s8, b=b8, c=None), 0)
    ref8 = oracle.gemm_ag(s8, b8, None, 1.0, 0.0, 1, "e4m3")
    assert np.array_equal(d8.cpu().numpy(), bf16_bits_of(ref8))
    # 64 K-steps of e4m3 (K = 4096) over every staging: still exact
    Ks, ms, Ns = 4096, 130, 264
    s8 = [gen.encode_e4m3(rng.integers(-4, 5, (ms, Ks)) * 0.25) for _ in range(2)]
    b8 = gen.encode_e4m3(rng.integers(-2, 3, (Ns, Ks)) * 0.5)
    c8 = gen.encode_bf16(rng.integers(-3, 4, (2 * ms, Ns)) * 0.5)
    case8 = W.AgCase("int8longk", M=2 * ms, N=Ns, K=Ks, P=2, rank=1, dtype="e4m3", alpha=1.0, beta=1.0)
    say("ag: integer exactness, K = 4096")
    ref8 = bf16_bits_of(oracle.gemm_ag(s8, b8, c8, 1.0, 1.0, 1, "e4m3"))
    for flags in (0, tp.UNSTAGED):
        d8 = run_ag(case8, dict(a_slices=s8, b=b8, c=c8), flags)
        assert np.array_equal(d8.cpu().numpy(), ref8), flags


def test_ag_beta_zero_never_reads_c():
    case = W.SMALL_AG[3]
    inp = W.ag_inputs(case)
    say("ag: beta=0 with NaN C")
    slices = [dev(s) for s in inp["a_slices"]]
    nan_c = bf16_empty(case.M, case.N)          # NaN everywhere
    d = bf16_empty(case.M, case.N)
    tp.stage_ag(slices, dev(inp["b"]), nan_c, d, M=case.M, N=case.N, K=case.K, dtype=tp.E4M3,
                alpha=1.0, beta=0.0)
    torch.cuda.synchronize()
    assert_parity(host_f64(d), oracle_ag(case, inp), "beta0")


def test_ag_graph_replay_sees_new_data():
    case = W.SMALL_AG[0]
    inp = W.ag_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    d = bf16_empty(case.M, case.N)
    kw = dict(M=case.M, N=case.N, K=case.K, rank=0, alpha=1.0, beta=1.0, flags=tp.FORCE_GRAPH)
    say("ag: graph replay with changed inputs")
    for it in range(3):
        tp.stage_ag(slices, b, c, d, **kw)      # same pointers: replays one graph
        torch.cuda.synchronize()
        ref = oracle.gemm_ag([s.cpu().numpy().view(np.uint16) for s in slices], inp["b"],
                             c.cpu().numpy().view(np.uint16), 1.0, 1.0, 0)
        assert_parity(host_f64(d), ref, f"replay {it}")
        for s in slices:                          # new slice contents in place
            s.copy_(torch.roll(s, 1, dims=0))
        c.copy_(torch.flip(c, dims=[0]))


def test_ag_empty_and_single_stage():
    say("ag: M=0 and P=1")
    b = torch.zeros((64, 64), dtype=torch.int16, device="cuda")
    d = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    s0 = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    tp.stage_ag([s0, s0.clone()], b, None, d, M=0, N=64, K=64, alpha=1.0, beta=0.0)
    case = W.AgCase("p1", M=136, N=72, K=264, P=1, dist="u11")
    inp = W.ag_inputs(case)
    d = run_ag(case, inp, 0)
    assert_parity(host_f64(d), oracle_ag(case, inp), "P=1")


@pytest.mark.parametrize("contiguous", [False, True])
def test_ag_stage_groups_are_bitwise_identical(contiguous):
    """Every grouping of the remote stages (one gate per stage, one gate for
    all, auto) and merged deliveries of adjacent slices give the same bits."""
    case = W.AgCase("groups", M=8 * 96, N=264, K=256, P=8, rank=5, dist="u11")
    inp = W.ag_inputs(case)
    if contiguous:      # all peer slices back to back in one allocation
        whole = dev(np.concatenate(inp["a_slices"], axis=0))
        slices = [whole[s * case.m:(s + 1) * case.m] for s in range(case.P)]
    else:
        slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    ref = oracle_ag(case, inp)
    outs = []
    for groups in (0, 1, 2, 3, 7, 9):
        for flags in (0, tp.FORCE_GRAPH, tp.NO_GRAPH, tp.NO_COPY, tp.COPY_SDMA):
            say(f"ag groups: contiguous={contiguous} groups={groups} flags={flags}")
            d = bf16_empty(case.M, case.N)
            tp.stage_ag(slices, b, c, d, M=case.M, N=case.N, K=case.K, rank=case.rank, alpha=1.0, beta=1.0,
                        flags=flags, groups=groups)
            torch.cuda.synchronize()
            outs.append(d.cpu())
    assert_parity(host_f64(d), ref, "groups")
    assert all(torch.equal(o, outs[0]) for o in outs)


# One launch over all rows (the unstaged call) whose 256 x 256 tiles would
# end in a partial round: 4096 x 4352 is 272 tiles on 256 CUs, so the
# launcher runs the first 4096 columns as one whole round and the last 256
# columns as a second launch of 128 x 256 tiles. Column offsets of B (both
# layouts), C and D must then land right.
ROUND_SPLIT = [
    W.AgCase("ag_bf16_round_split", M=4096, N=4352, K=256, P=2, rank=1, dist="u11", alpha=0.5, beta=1.0),
    W.AgCase("ag_bf16_kn_round_split", M=4096, N=4352, K=192, P=2, rank=0, b_layout="kn", beta=-1.0),
    W.AgCase("ag_e4m3_round_split", M=4096, N=4352, K=384, P=2, rank=1, dtype="e4m3", dist="n05",
             c_dist="n01"),
    # a ragged last tile-row (4000 rows: 16 tile-rows of 256, the last 160
    # rows deep) and a ragged remainder (4344 columns: 248 after the split)
    W.AgCase("ag_bf16_round_split_ragged", M=4000, N=4344, K=256, P=2, rank=0, dist="u11", beta=1.0),
]


@pytest.mark.parametrize("case", ROUND_SPLIT, ids=lambda c: c.name)
def test_ag_round_split_launch(case):
    inp = W.ag_inputs(case)
    ref = oracle_ag(case, inp)
    outs = {}
    for name in ("unstaged", "default"):
        say(f"ag: {case.name} mode={name}")
        d = run_ag(case, inp, MODES[name])
        assert_parity(host_f64(d), ref, f"{case.name}/{name}")
        outs[name] = d.cpu()
    assert torch.equal(outs["unstaged"], outs["default"])
