"""Calls recorded into the caller's own graph: the caller captures its stream
(torch.cuda.graph) around an eager library call that fans out over the
library's internal streams, then replays the graph. The call must then
join its internal streams to the capture with events (stream memory
operations on static words would not be recorded, and a replay would
repeat their stamped values). Each replay follows new input data written
in place, an eager call on the same data (the reference) and a
synchronisation, and must equal that eager call bit for bit."""
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

REPLAYS = 3


def record(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def refill(tensors, seed):
    """New bf16 data of the same scale in place (small values: no overflow)."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    for t in tensors:
        v = (torch.rand(t.shape, device="cuda", generator=gen) - 0.5).to(torch.bfloat16)
        t.copy_(v.view(torch.int16))


def replay_against_eager(name, g, eager, out, ref_out, inputs):
    for rep in range(REPLAYS):
        refill(inputs, 100 + rep)
        eager()
        torch.cuda.synchronize()
        say(f"caller graph: {name} replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"{name}: replay {rep} differs from the eager call"


AG_CASES = [
    (W.AgCase("capture_ag_bf16_p2", M=2 * 512, N=1024, K=512, P=2, rank=1, dist="u11"), 0),
    (W.AgCase("capture_ag_bf16_p4_three_runs", M=4 * 256, N=512, K=1024, P=4, rank=2, dist="u11"), 3),
]


@pytest.mark.parametrize("case,groups", AG_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_staged_all_gather_in_caller_graph(case, groups):
    assert 2.0 * case.M * case.N * case.K >= 1e9       # staged over several streams
    inp = W.ag_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, alpha=case.alpha, beta=case.beta, groups=groups)
    probe = bf16_empty(case.M, case.N)
    ws = torch.empty(tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, probe, **kw)), dtype=torch.uint8,
                     device="cuda")
    d, d_ref = bf16_empty(case.M, case.N), bf16_empty(case.M, case.N)
    tp.stage_ag(slices, b, c, d_ref, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert_parity(host_f64(d_ref), oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta,
                                                  case.rank), case.name)
    g = record(lambda: tp.stage_ag(slices, b, c, d, workspace=ws, **kw))
    replay_against_eager(case.name, g, lambda: tp.stage_ag(slices, b, c, d_ref, workspace=ws, **kw), d, d_ref,
                         slices + [b, c])


def test_staged_all_gather_noalloc_in_caller_graph():
    """The allocation-free entry point, whose callers include code under
    stream capture."""
    case = AG_CASES[0][0]
    inp = W.ag_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, alpha=case.alpha, beta=case.beta)
    d, d_ref = bf16_empty(case.M, case.N), bf16_empty(case.M, case.N)
    tp.stage_ag_noalloc(slices, b, c, d_ref, **kw)      # eager first: the library's set-up is done
    torch.cuda.synchronize()
    assert_parity(host_f64(d_ref), oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta,
                                                  case.rank), "noalloc")
    g = record(lambda: tp.stage_ag_noalloc(slices, b, c, d, **kw))
    replay_against_eager("noalloc", g, lambda: tp.stage_ag_noalloc(slices, b, c, d_ref, **kw), d, d_ref,
                         slices + [b, c])


def test_staged_reduce_scatter_in_caller_graph():
    case = W.RsCase("capture_rs_bf16_p4", M=4 * 256, N=1024, K=512, P=4, rank=1, std=0.5)
    inp = W.rs_inputs(case)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    kw = dict(M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank)
    probe = bf16_empty(case.M, case.N)
    ws = torch.empty(max(tp.stage_rs_workspace_size(tp.rs_args(a, b, inc, probe, **kw)), 1), dtype=torch.uint8,
                     device="cuda")
    d, d_ref = bf16_empty(case.M, case.N), bf16_empty(case.M, case.N)
    tp.stage_rs(a, b, inc, d_ref, workspace=ws, **kw)
    torch.cuda.synchronize()
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], 1.0, case.rank, case.P)
    for blk in range(case.P):
        rows = slice(blk * case.m, (blk + 1) * case.m)
        assert_parity(host_f64(d_ref)[rows], ref[rows], f"block {blk}")
    g = record(lambda: tp.stage_rs(a, b, inc, d, workspace=ws, **kw))
    replay_against_eager(case.name, g, lambda: tp.stage_rs(a, b, inc, d_ref, workspace=ws, **kw), d, d_ref,
                         [a, b] + [x for x in inc if x is not None])


def test_ffn_in_caller_graph():
    case = W.SMALL_FFN[0]
    inp = W.ffn_inputs(case)
    t = {k: dev(v) for k, v in inp.items()}
    args = (t["x"], t["w1"], t["b1"], t["wout"], t["bout"], t["gx"], t["bx"], t["gg"], t["bg"])
    kw = dict(PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps)
    y, y_ref = bf16_empty(case.PB, case.L, case.D), bf16_empty(case.PB, case.L, case.D)
    ws = torch.empty(max(tp.ffn_slot_forward_workspace_size(tp.ffn_args(*args, y, **kw)), 1), dtype=torch.uint8,
                     device="cuda")
    tp.ffn_slot_forward(*args, y_ref, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert_parity(host_f64(y_ref), oracle.ffn_slot_forward(inp, case.eps), case.name)
    g = record(lambda: tp.ffn_slot_forward(*args, y, workspace=ws, **kw))
    # new activations only: the weights and LayerNorm parameters keep their scale
    replay_against_eager(case.name, g, lambda: tp.ffn_slot_forward(*args, y_ref, workspace=ws, **kw), y, y_ref,
                         [t["x"]])
