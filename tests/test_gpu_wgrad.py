"""GPU parity of the staged weight gradient (tpgemm_stage_wgrad) against the
oracle, through the C ABI: every issue mode and stage grouping, both gathered
operands, the ring wrap of the local operand, held deliveries, integer-exact
inputs, the empty contraction and the composed backward of the all-gather
linear."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import gen
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64, bf16_bits_of
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

MODES = {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "unstaged": tp.UNSTAGED,
         "no_copy": tp.NO_COPY, "serial": tp.SERIAL_STAGES, "sdma": tp.COPY_SDMA, "shader": tp.COPY_SHADER}


def gathered_of(case):
    return tp.GATHER_X if case.gathered == "x" else tp.GATHER_G


def run(case, inp, flags=0, groups=0, workspace=None, local=None, slices=None):
    local = dev(inp["local"]) if local is None else local
    if slices is None and (flags & tp.NO_COPY) and (groups == 0 or flags & tp.UNSTAGED):
        _, slices = contiguous_slices(inp)      # one launch in place needs the slices in one buffer
    slices = [dev(s) for s in inp["slices"]] if slices is None else slices
    d = bf16_empty(case.N, case.K)
    tp.stage_wgrad(local, slices, d, M=case.M, N=case.N, K=case.K, rank=case.rank, gathered=gathered_of(case),
                   alpha=case.alpha, flags=flags, groups=groups, workspace=workspace)
    torch.cuda.synchronize()
    return d


def contiguous_slices(inp):
    """The slices as views of one buffer in rank order (for in-place unstaged calls)."""
    big = dev(np.concatenate(inp["slices"], axis=0))
    m = inp["slices"][0].shape[0]
    return big, [big[s * m:(s + 1) * m] for s in range(len(inp["slices"]))]


@pytest.mark.parametrize("case", W.SMALL_WGRAD, ids=lambda c: c.name)
def test_wgrad_parity_all_modes(case):
    """Every issue mode, both with the library's choice (one gathered launch)
    and staged (groups >= 1)."""
    inp = W.wgrad_inputs(case)
    ref = oracle.wgrad_staged(inp["local"], inp["slices"], case.gathered, case.rank, case.alpha)
    outs = {}
    for name, flags in MODES.items():
        for groups in (0, 1):
            say(f"wgrad: {case.name} mode={name} groups={groups}")
            outs[name, groups] = run(case, inp, flags, groups)
            assert_parity(host_f64(outs[name, groups]), ref, f"{case.name}/{name}/{groups}")
    for groups in sorted({2, case.P - 1}):
        if groups > case.P - 1:
            continue
        say(f"wgrad: {case.name} groups={groups}")
        d = run(case, inp, 0, groups)
        assert_parity(host_f64(d), ref, f"{case.name}/groups={groups}")
    say(f"wgrad: {case.name} unstaged in place")
    _, sl = contiguous_slices(inp)
    d = run(case, inp, tp.UNSTAGED | tp.NO_COPY, slices=sl)
    assert_parity(host_f64(d), ref, f"{case.name}/unstaged in place")
    # the same launches give the same bits whatever the issue mode
    for name in ("graph", "eager", "serial", "sdma", "shader"):
        assert torch.equal(outs[name, 1], outs["default", 1]), name
        assert torch.equal(outs[name, 0], outs["default", 0]), name
    assert torch.equal(outs["unstaged", 1], outs["default", 0])
    assert torch.equal(d, outs["default", 0])


def test_wgrad_integer_inputs_are_exact():
    """Small-integer operands: every fp32 partial sum is exact, so each mode's
    result is the oracle's value rounded once to bf16, bit for bit."""
    case = W.WgCase("wg_int", M=8 * 64, N=264, K=200, P=8, rank=6)
    rng = np.random.default_rng(11)
    inp = dict(local=gen.encode_bf16(rng.integers(-3, 4, size=(case.M, case.N)).astype(np.float64)),
               slices=[gen.encode_bf16(rng.integers(-3, 4, size=(case.m, case.K)).astype(np.float64))
                       for _ in range(case.P)])
    ref_bits = bf16_bits_of(oracle.wgrad_staged(inp["local"], inp["slices"], "x", case.rank))
    for name, flags in MODES.items():
        for groups in (0, 3):
            say(f"wgrad int: mode={name} groups={groups}")
            d = run(case, inp, flags, groups)
            assert np.array_equal(d.cpu().numpy(), ref_bits), (name, groups)


def test_wgrad_waits_for_held_deliveries():
    """Deliveries held behind a host sleep, receive slots and the fp32 partial
    poisoned with NaN: every gated launch still reads only landed slices."""
    hold = tp.DEBUG_HOLD_DELIVERIES
    for case in (W.SMALL_WGRAD[0], W.SMALL_WGRAD[1]):
        inp = W.wgrad_inputs(case)
        ref = oracle.wgrad_staged(inp["local"], inp["slices"], case.gathered, case.rank, case.alpha)
        for flags, groups in [(hold, 1), (hold, case.P - 1), (hold | tp.COPY_SDMA, 2), (hold | tp.UNSTAGED, 0)]:
            say(f"wgrad hold: {case.name} flags={flags} groups={groups}")
            ws = torch.full((16 << 20,), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint8)
            d = run(case, inp, flags, groups, workspace=ws)
            got = host_f64(d)
            assert not np.isnan(got).any()
            assert_parity(got, ref, f"{case.name} hold {flags}/{groups}")


def test_wgrad_empty_contraction_writes_zeros():
    local = torch.empty((0, 64), dtype=torch.int16, device="cuda")
    slices = [torch.empty((0, 40), dtype=torch.int16, device="cuda") for _ in range(4)]
    d = bf16_empty(64, 40)
    tp.stage_wgrad(local, slices, d, M=0, N=64, K=40, rank=1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(d).item() == 0


def test_all_gather_linear_backward():
    """The composed backward of Y = X_g W^T on one rank: dX (this rank's own
    block) from the reduce-scatter call with W read in the (K, N) layout and
    the peers' partials incoming; dW from the weight-gradient call with X
    gathered. Against the oracle's two forms."""
    P, m, N, K, rank = 4, 128, 264, 320, 2
    M = P * m
    key = lambda tag, r=rank: gen.stream_key(77 + r, tag)
    dy = gen.normal_bf16(key("dy"), (M, N))
    w = gen.normal_bf16(key("w"), (N, K), 0.0, 0.05)
    xs = [gen.normal_bf16(key("x", s), (m, K)) for s in range(P)]
    incoming = [None if j == rank else gen.normal_bf16(key("inc", j), (m, K)) for j in range(P)]
    dxg = bf16_empty(M, K)
    say("backward: dgrad")
    tp.stage_rs(dev(dy), dev(w), [dev(x) for x in incoming], dxg, M=M, N=K, K=N, P=P, rank=rank, b_layout=tp.B_KN)
    dw = bf16_empty(N, K)
    say("backward: wgrad")
    tp.stage_wgrad(dev(dy), [dev(x) for x in xs], dw, M=M, N=N, K=K, rank=rank)
    torch.cuda.synchronize()
    ref_dx = oracle.gemm_rs(dy, w, incoming, 1.0, rank, P, b_layout="kn")
    assert_parity(host_f64(dxg)[rank * m:(rank + 1) * m], ref_dx[rank * m:(rank + 1) * m], "dX own block")
    assert_parity(host_f64(dw), oracle.wgrad_staged(dy, xs, "x", rank), "dW")


def test_wgrad_graph_replay_sees_new_data():
    """A recorded call replayed three times with new operand contents in
    place and eager work between the replays: every replay matches the eager
    call on the same data."""
    case = W.SMALL_WGRAD[2]
    inp = W.wgrad_inputs(case)
    local, slices = dev(inp["local"]), [dev(s) for s in inp["slices"]]
    d = bf16_empty(case.N, case.K)
    e = bf16_empty(case.N, case.K)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for groups in (0, 1):
        for it in range(3):
            say(f"wgrad: graph replay {it} groups={groups}")
            kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, groups=groups, workspace=ws)
            tp.stage_wgrad(local, slices, d, flags=tp.FORCE_GRAPH, **kw)
            torch.cuda.synchronize()
            tp.stage_wgrad(local, slices, e, flags=tp.NO_GRAPH, **kw)
            torch.cuda.synchronize()
            assert torch.equal(d, e), it
            local.copy_(torch.roll(local, 1, dims=0))      # new contents in place
            for s in slices:
                s.copy_(torch.flip(s, dims=[1]))
