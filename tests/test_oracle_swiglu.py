"""Pins of the oracle's SwiGLU TP block share (CPU)."""
import math

import numpy as np
import torch

import oracle
from synth import workloads as W


def test_swiglu_brute_force_tiny():
    case = W.SwigluCase("t", S=2, D=3, F=2, P=2, std=0.7)
    inp = W.swiglu_inputs(case)
    X = np.concatenate([oracle.decode_bf16(s) for s in inp["x_shards"]])
    w13 = oracle.decode_bf16(inp["w13"])
    w2 = oracle.decode_bf16(inp["w2"])
    out = oracle.swiglu_block(inp["x_shards"], inp["w13"], inp["w2"])
    for i in range(4):
        h = []
        for f in range(2):
            u = sum(X[i, d] * w13[d, f] for d in range(3))
            v = sum(X[i, d] * w13[d, 2 + f] for d in range(3))
            h.append(u / (1 + math.exp(-u)) * v)
        for j in range(3):
            assert abs(out[i, j] - sum(h[f] * w2[f, j] for f in range(2))) < 1e-12


def test_swiglu_matches_torch_and_rank_order():
    case = W.SMALL_SWIGLU[0]
    inp = W.swiglu_inputs(case)
    xs = [torch.from_numpy(oracle.decode_bf16(s)) for s in inp["x_shards"]]
    w13 = torch.from_numpy(oracle.decode_bf16(inp["w13"]))
    w2 = torch.from_numpy(oracle.decode_bf16(inp["w2"]))
    x = torch.cat(xs, 0)
    F = case.F
    ref = (torch.nn.functional.silu(x @ w13[:, :F]) * (x @ w13[:, F:])) @ w2
    got = oracle.swiglu_block(inp["x_shards"], inp["w13"], inp["w2"])
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-11)
    # rows of block s come from shard s (rank-major row order)
    S = case.S
    for s in range(case.P):
        part = (torch.nn.functional.silu(xs[s] @ w13[:, :F]) * (xs[s] @ w13[:, F:])) @ w2
        np.testing.assert_allclose(got[s * S:(s + 1) * S], part.numpy(), rtol=1e-11, atol=1e-11)
    rows = [0, S - 1, S, 3 * S + 5]
    np.testing.assert_allclose(oracle.swiglu_hidden_rows(inp["x_shards"], inp["w13"], rows),
                               oracle.swiglu_hidden(inp["x_shards"], inp["w13"])[rows], rtol=1e-13, atol=1e-13)
