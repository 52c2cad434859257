"""GPU parity of the per-slot FFN backward (ffn_slot_backward) against the
oracle, through the C ABI: every gradient (input, both weights, both biases,
the four LayerNorm parameters) on small cases with ragged tiles, the affine
LayerNorm and large biases; deterministic across runs; the empty batch.

Tolerance: the p04 statement's backward rule for bf16, a per-gradient
Frobenius relative error of at most 2e-2 (denominator clamped at 1e-12)."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64

pytestmark = pytest.mark.gpu

BWD_TOL = 2e-2

CASES = [W.FfnCase("ffnb_p2_d200_k2", B=32, T=4, D=200, k=2, P=2, affine=True, big_bias=True),
         W.FfnCase("ffnb_p4_d256_k3", B=32, T=8, D=256, k=3, P=4),
         W.FfnCase("ffnb_p8_d128_k6", B=16, T=24, D=128, k=6, P=8, affine=True, rank=3)]

SHAPES = lambda c: dict(dx=(c.PB, c.L, c.D), dw1=(c.L, c.D, 2 * c.H), db1=(c.L, 2 * c.H), dwout=(c.L, c.H, c.D),
                        dbout=(c.L, c.D), dgx=(c.H,), dbx=(c.H,), dgg=(c.H,), dbg=(c.H,))
ORACLE_KEY = dict(dx="x", dw1="w1", db1="b1", dwout="wout", dbout="bout", dgx="gx", dbx="bx", dgg="gg", dbg="bg")


def run_backward(case, inp, dy, flags=0):
    t = {k: dev(v) for k, v in inp.items()}
    grads = {k: bf16_empty(*shape) for k, shape in SHAPES(case).items()}
    tp.ffn_slot_backward(t["x"], t["w1"], t["b1"], t["wout"], t["gx"], t["bx"], t["gg"], t["bg"], dev(dy), grads,
                         PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps, flags=flags)
    torch.cuda.synchronize()
    return grads


def fro(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-12))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_ffn_backward_parity(case):
    inp = W.ffn_inputs(case)
    dy = W.ffn_upstream_grad(case)
    say(f"ffn backward: {case.name} PB={case.PB} L={case.L} D={case.D} H={case.H}")
    grads = run_backward(case, inp, dy)
    ref = oracle.ffn_slot_backward(inp, dy, case.eps)
    errs = {k: fro(host_f64(g), ref[ORACLE_KEY[k]]) for k, g in grads.items()}
    say(f"ffn backward: {case.name} frobenius {errs}")
    assert all(e <= BWD_TOL for e in errs.values()), errs
    again = run_backward(case, inp, dy)
    serial = run_backward(case, inp, dy, tp.SERIAL_STAGES)
    graph = run_backward(case, inp, dy, tp.FORCE_GRAPH)
    for k in grads:                      # fixed reduction order: the same bits every run and issue mode
        assert torch.equal(grads[k], again[k]), k
        assert torch.equal(grads[k], serial[k]), k
        assert torch.equal(grads[k], graph[k]), k


def test_ffn_backward_empty_batch_zeroes_parameter_grads():
    case = W.FfnCase("ffnb_empty", B=0, T=4, D=64, k=2, P=2)
    grads = {k: bf16_empty(*shape) for k, shape in SHAPES(case).items()}
    z = torch.zeros(1 << 16, dtype=torch.int16, device="cuda")
    say("ffn backward: empty batch")
    tp.ffn_slot_backward(z, z, z, z, z, z, z, z, z, grads, PB=0, L=case.L, D=case.D, H=case.H)
    torch.cuda.synchronize()
    for k, g in grads.items():
        if k != "dx":
            assert torch.count_nonzero(g).item() == 0, k


def test_ffn_backward_graph_replay_sees_new_data():
    """The recorded backward replayed three times with a new upstream gradient
    in place and eager work between: each replay equals the eager call."""
    case = CASES[1]
    inp = W.ffn_inputs(case)
    t = {k: dev(v) for k, v in inp.items()}
    dy = dev(W.ffn_upstream_grad(case))
    g_rep = {k: bf16_empty(*shape) for k, shape in SHAPES(case).items()}
    g_eag = {k: bf16_empty(*shape) for k, shape in SHAPES(case).items()}
    ws = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    args = (t["x"], t["w1"], t["b1"], t["wout"], t["gx"], t["bx"], t["gg"], t["bg"], dy)
    kw = dict(PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps, workspace=ws)
    for it in range(3):
        say(f"ffn backward: graph replay {it}")
        tp.ffn_slot_backward(*args, g_rep, flags=tp.FORCE_GRAPH, **kw)
        torch.cuda.synchronize()
        tp.ffn_slot_backward(*args, g_eag, flags=tp.NO_GRAPH, **kw)
        torch.cuda.synchronize()
        for k in g_rep:
            assert torch.equal(g_rep[k], g_eag[k]), (it, k)
        dy.copy_(torch.roll(dy, 1, dims=0))
