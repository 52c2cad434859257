"""Pins of the oracle's dispatch / combine permutes (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dispatch_p2_b1_t2_d1.json")


def test_worked_example_from_the_statement():
    g = json.load(open(GOLDEN))
    inputs = [np.array(x, dtype=np.int64) for x in g["inputs"]]
    for r in range(g["P"]):
        got = oracle.dispatch(inputs, r)
        assert got.shape == (2, 1, 1)
        assert np.array_equal(got, np.array(g["dispatched"][r]))
    # identity local compute: combine restores each rank's input
    ys = [oracle.dispatch(inputs, r) for r in range(g["P"])]
    for r in range(g["P"]):
        assert np.array_equal(oracle.combine(ys, r), inputs[r])


@pytest.mark.parametrize("P,B,T,D", [(1, 3, 16, 128), (2, 4, 16, 128), (4, 5, 32, 136), (8, 2, 64, 200)])
def test_dispatch_combine_round_trip_all_ranks(P, B, T, D):
    src = W.permute_sources(B, T, D, P, dtype="u8")
    ys = [oracle.dispatch(src, r) for r in range(P)]
    for r in range(P):
        assert ys[r].shape == (P * B, T // P, D)
        assert np.array_equal(oracle.combine(ys, r), src[r])
    if P == 1:
        assert np.array_equal(ys[0], src[0])


def test_dispatch_index_map():
    P, B, T, D = 4, 3, 8, 5
    L = T // P
    src = [np.arange(B * T * D).reshape(B, T, D) + 1000 * s for s in range(P)]
    for r in range(P):
        out = oracle.dispatch(src, r)
        for s in range(P):
            for b in range(B):
                for l in range(L):
                    assert np.array_equal(out[s * B + b, l], src[s][b, r * L + l])
