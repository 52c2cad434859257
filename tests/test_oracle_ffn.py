"""Pins of the oracle's per-token-slot FFN (CPU).

Closed forms of LayerNorm and SiLU, scalar brute force on tiny shapes, and an
independent implementation from library routines (torch float64 layer_norm,
silu, matmul) on the public development shape of the p04 statement.
Planted mistakes (in a copy of the oracle's helpers) must fail these pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.ffn as offn
from synth import workloads as W


def test_layer_norm_constant_row_gives_beta():
    v = np.full((3, 10), 7.25)
    beta = np.linspace(-1, 1, 10)
    np.testing.assert_array_equal(oracle.layer_norm(v, np.full(10, 3.0), beta, 1e-5), np.tile(beta, (3, 1)))


def test_layer_norm_plus_minus_row():
    a = 0.37
    v = np.array([[a, -a] * 8])
    got = oracle.layer_norm(v, np.ones(16), np.zeros(16), 1e-5)
    want = np.array([[a, -a] * 8]) / math.sqrt(a * a + 1e-5)
    np.testing.assert_allclose(got, want, rtol=1e-15)


def test_layer_norm_moments_and_library():
    rng = np.random.default_rng(0)
    v = rng.normal(3.0, 2.0, (64, 333))
    y = oracle.layer_norm(v, np.ones(333), np.zeros(333), 1e-5)
    var = v.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    g, b = rng.uniform(0.5, 1.5, 333), rng.uniform(-.5, .5, 333)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(v), (333,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(v, g, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_silu_identities_and_library():
    x = np.linspace(-50, 50, 2001)
    s = oracle.silu(x)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - oracle.silu(-x), x, atol=1e-12)
    np.testing.assert_allclose(s, torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    assert np.isfinite(oracle.silu(np.array([-1000.0, 1000.0]))).all()


def brute_ffn(inp, eps=1e-5):
    """Literal scalar loops, math module only."""
    d = lambda a: oracle.decode_bf16(a).tolist()
    X, w1, b1, wo, bo = d(inp["x"]), d(inp["w1"]), d(inp["b1"]), d(inp["wout"]), d(inp["bout"])
    gx, bx, gg, bg = d(inp["gx"]), d(inp["bx"]), d(inp["gg"]), d(inp["bg"])
    PB, L, D = len(X), len(X[0]), len(X[0][0])
    H = len(gx)
    Y = np.zeros((PB, L, D))
    for n in range(PB):
        for l in range(L):
            z = [sum(X[n][l][i] * w1[l][i][j] for i in range(D)) + b1[l][j] for j in range(2 * H)]
            def ln(v, g, b):
                mu = sum(v) / len(v)
                var = sum((t - mu) ** 2 for t in v) / len(v)
                return [(t - mu) / math.sqrt(var + eps) * g[i] + b[i] for i, t in enumerate(v)]
            u = ln(z[:H], gx, bx)
            g = ln(z[H:], gg, bg)
            h = [u[i] * (g[i] / (1 + math.exp(-g[i]))) for i in range(H)]
            for j in range(D):
                Y[n, l, j] = sum(h[i] * wo[l][i][j] for i in range(H)) + bo[l][j]
    return Y


TINY = W.FfnCase("tiny", B=1, T=2, D=4, k=2, P=2, affine=True, big_bias=True)


def test_ffn_matches_brute_force_tiny():
    inp = W.ffn_inputs(TINY)
    np.testing.assert_allclose(oracle.ffn_slot_forward(inp), brute_ffn(inp), rtol=1e-12, atol=1e-12)


def torch_ffn(inp, eps=1e-5):
    t = {k: torch.from_numpy(oracle.decode_bf16(v)) for k, v in inp.items()}
    H = t["wout"].shape[1]
    outs = []
    for l in range(t["x"].shape[1]):
        z = torch.matmul(t["x"][:, l, :], t["w1"][l]) + t["b1"][l]
        u = torch.nn.functional.layer_norm(z[:, :H], (H,), t["gx"], t["bx"], eps)
        g = torch.nn.functional.layer_norm(z[:, H:], (H,), t["gg"], t["bg"], eps)
        outs.append(torch.matmul(u * torch.nn.functional.silu(g), t["wout"][l]) + t["bout"][l])
    return torch.stack(outs, dim=1).numpy()


@pytest.mark.parametrize("case", W.SMALL_FFN, ids=lambda c: c.name)
def test_ffn_matches_torch_library(case):
    inp = W.ffn_inputs(case)
    np.testing.assert_allclose(oracle.ffn_slot_forward(inp), torch_ffn(inp), rtol=1e-10, atol=1e-10)


def test_ffn_rows_match_full():
    inp = W.ffn_inputs(W.SMALL_FFN[1])
    full = oracle.ffn_slot_forward(inp)
    pairs = [(0, 0), (5, 3), (23, 2), (11, 1)]
    np.testing.assert_allclose(oracle.ffn_slot_rows(inp, pairs), np.stack([full[n, l] for n, l in pairs]),
                               rtol=1e-12, atol=1e-12)


def test_ffn_single_slot_is_plain_ffn():
    # L = 1, P = 1: the block reduces to LN/SiLU-gated FFN on [B, D] rows
    case = W.FfnCase("l1", B=3, T=1, D=8, k=2, P=1, affine=True, big_bias=True)
    inp = W.ffn_inputs(case)
    np.testing.assert_allclose(oracle.ffn_slot_forward(inp), brute_ffn(inp), rtol=1e-12, atol=1e-12)


# ---- planted mistakes: each must be caught by the brute-force pin ----------
def _sample_var_ln(v, gamma, beta, eps):
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).sum(axis=-1, keepdims=True) / (v.shape[-1] - 1)
    return (v - mu) / np.sqrt(var + eps) * gamma + beta


def _no_mean_ln(v, gamma, beta, eps):
    var = (v ** 2).mean(axis=-1, keepdims=True)
    return v / np.sqrt(var + eps) * gamma + beta


def _sigmoid_gate(t):
    return 1.0 / (1.0 + np.exp(-t))


@pytest.mark.parametrize("attr,bad", [("layer_norm", _sample_var_ln), ("layer_norm", _no_mean_ln),
                                      ("silu", _sigmoid_gate)])
def test_planted_mistakes_are_caught(monkeypatch, attr, bad):
    inp = W.ffn_inputs(TINY)
    ref = brute_ffn(inp)
    monkeypatch.setattr(offn, attr, bad)
    assert not np.allclose(offn.ffn_slot_forward(inp), ref, rtol=1e-6, atol=1e-6)


def test_planted_swapped_halves_caught(monkeypatch):
    inp = W.ffn_inputs(TINY)
    ref = brute_ffn(inp)
    orig = offn._slot_rows

    def swapped(xrows, l, q, H, eps):
        q2 = dict(q)
        q2["w1"] = np.concatenate([q["w1"][:, :, H:], q["w1"][:, :, :H]], axis=2)
        q2["b1"] = np.concatenate([q["b1"][:, H:], q["b1"][:, :H]], axis=1)
        return orig(xrows, l, q2, H, eps)
    monkeypatch.setattr(offn, "_slot_rows", swapped)
    assert not np.allclose(offn.ffn_slot_forward(inp), ref, rtol=1e-6, atol=1e-6)
