"""GPU parity of dispatch_permute / combine_permute: bit-exact against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dispatch_p2_b1_t2_d1.json")


def test_worked_example_int64():
    g = json.load(open(GOLDEN))
    say("permute: worked example P=2 B=1 T=2 D=1")
    srcs = [torch.tensor(x, dtype=torch.int64, device="cuda") for x in g["inputs"]]
    outs = []
    for r in range(2):
        out = torch.full((2, 1, 1), -1, dtype=torch.int64, device="cuda")
        tp.dispatch_permute(srcs, out, rank=r, B=1, T=2, D=1, elem_bytes=8)
        outs.append(out)
    torch.cuda.synchronize()
    for r in range(2):
        assert outs[r].cpu().tolist() == g["dispatched"][r]
    for r in range(2):
        back = torch.full((1, 2, 1), -1, dtype=torch.int64, device="cuda")
        tp.combine_permute(outs, back, rank=r, B=1, T=2, D=1, elem_bytes=8)
        torch.cuda.synchronize()
        assert back.cpu().tolist() == g["inputs"][r]


@pytest.mark.parametrize("P,B,T,D,dtype", [(1, 3, 16, 128, "bf16"), (2, 4, 16, 128, "bf16"),
                                           (4, 5, 32, 136, "bf16"), (8, 2, 64, 200, "u8"),
                                           (4, 3, 16, 131, "u8"), (8, 7, 64, 1280, "bf16")])
def test_round_trip_all_ranks(P, B, T, D, dtype):
    say(f"permute: round trip P={P} B={B} T={T} D={D} {dtype}")
    src = W.permute_sources(B, T, D, P, dtype=dtype)
    eb = 2 if dtype == "bf16" else 1
    tdt = torch.int16 if eb == 2 else torch.uint8
    view = np.int16 if eb == 2 else np.uint8
    dsrc = [torch.from_numpy(s.view(view)).cuda() for s in src]
    ys = []
    for r in range(P):
        y = torch.zeros((P * B, T // P, D), dtype=tdt, device="cuda")
        tp.dispatch_permute(dsrc, y, rank=r, B=B, T=T, D=D, elem_bytes=eb)
        ys.append(y)
    torch.cuda.synchronize()
    for r in range(P):
        assert np.array_equal(ys[r].cpu().numpy().view(src[0].dtype), oracle.dispatch(src, r))
    for r in range(P):
        back = torch.zeros((B, T, D), dtype=tdt, device="cuda")
        tp.combine_permute(ys, back, rank=r, B=B, T=T, D=D, elem_bytes=eb)
        torch.cuda.synchronize()
        assert np.array_equal(back.cpu().numpy().view(src[0].dtype), src[r])


def test_empty_is_a_no_op():
    src = [torch.zeros((0, 8, 16), dtype=torch.int16, device="cuda") for _ in range(2)]
    out = torch.zeros((0, 4, 16), dtype=torch.int16, device="cuda")
    tp.dispatch_permute(src, out, rank=1, B=0, T=8, D=16, elem_bytes=2)
    torch.cuda.synchronize()


@pytest.mark.slow
def test_full_ffn_workload_shapes():
    """8 sources [512, 64, 1280] bf16 (the FFN workload), every rank, bit-exact."""
    P, B, T, D = 8, 512, 64, 1280
    say("permute: full workload shapes")
    src = W.permute_sources(B, T, D, P)
    dsrc = [torch.from_numpy(s.view(np.int16)).cuda() for s in src]
    for r in (0, 5):
        y = torch.zeros((P * B, T // P, D), dtype=torch.int16, device="cuda")
        tp.dispatch_permute(dsrc, y, rank=r, B=B, T=T, D=D, elem_bytes=2)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), oracle.dispatch(src, r))
        back = torch.zeros((B, T, D), dtype=torch.int16, device="cuda")
        ys = [y if s == r else torch.from_numpy(oracle.dispatch(src, s).view(np.int16)).cuda() for s in range(P)]
        tp.combine_permute(ys, back, rank=r, B=B, T=T, D=D, elem_bytes=2)
        torch.cuda.synchronize()
        assert np.array_equal(back.cpu().numpy().view(np.uint16), src[r])
