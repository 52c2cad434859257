"""Pins of the oracle's FFN backward (CPU): every gradient against central
finite differences of the forward oracle (float64, a random direction per
parameter), which shares none of the backward's formulas; plus invariants
of the LayerNorm backward."""
import numpy as np
import pytest

import oracle
from oracle import ffn as F


def params(rng, L, D, H, affine=True):
    q = dict(w1=rng.normal(0, 0.5, (L, D, 2 * H)), b1=rng.normal(0, 0.5, (L, 2 * H)),
             wout=rng.normal(0, 0.5, (L, H, D)), bout=rng.normal(0, 0.5, (L, D)))
    if affine:
        q.update(gx=rng.uniform(0.5, 1.5, H), bx=rng.uniform(-0.5, 0.5, H),
                 gg=rng.uniform(0.5, 1.5, H), bg=rng.uniform(-0.5, 0.5, H))
    else:
        q.update(gx=np.ones(H), bx=np.zeros(H), gg=np.ones(H), bg=np.zeros(H))
    return q


@pytest.mark.parametrize("affine", [True, False])
def test_backward_matches_finite_differences(affine):
    rng = np.random.default_rng(5 + affine)
    PB, L, D, H, eps = 3, 2, 4, 8, 1e-5
    X = rng.normal(0, 1, (PB, L, D))
    q = params(rng, L, D, H, affine)
    dY = rng.normal(0, 1, (PB, L, D))
    g = F.backward_f64(X, q, dY, eps)
    loss = lambda X_, q_: float(np.sum(dY * F.forward_f64(X_, q_, eps)))
    step = 1e-6
    for key in ["x"] + list(q):
        V = rng.normal(0, 1, X.shape if key == "x" else q[key].shape)
        if key == "x":
            fd = (loss(X + step * V, q) - loss(X - step * V, q)) / (2 * step)
        else:
            qp, qm = dict(q), dict(q)
            qp[key], qm[key] = q[key] + step * V, q[key] - step * V
            fd = (loss(X, qp) - loss(X, qm)) / (2 * step)
        an = float(np.sum(g[key] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


def test_layer_norm_backward_invariants():
    """The input gradient of a LayerNorm sums to zero over a row and is
    orthogonal to the normalised row (the output is invariant to shifts and,
    through the variance, to scaling of the input)."""
    rng = np.random.default_rng(9)
    eps = 1e-5
    v = rng.normal(0, 2, (5, 16))
    xhat, r = F._ln_parts(v, eps)
    dxh = rng.normal(0, 1, (5, 16))
    dv = F._ln_backward(dxh, xhat, r)
    np.testing.assert_allclose(dv.sum(axis=1), 0, atol=1e-12)
    # orthogonality to xhat holds up to the eps term: the sum equals
    # r * eps / (var + eps) * sum(dxh * xhat), with var the row's variance
    var = v.var(axis=1)
    expect = r[:, 0] * eps / (var + eps) * (dxh * xhat).sum(axis=1)
    np.testing.assert_allclose((dv * xhat).sum(axis=1), expect, rtol=1e-6, atol=1e-14)


def test_zero_upstream_gradient_gives_zero():
    rng = np.random.default_rng(3)
    PB, L, D, H = 2, 2, 4, 8
    g = F.backward_f64(rng.normal(0, 1, (PB, L, D)), params(rng, L, D, H), np.zeros((PB, L, D)), 1e-5)
    assert all(np.count_nonzero(v) == 0 for v in g.values())


def test_bias_gradient_is_the_row_sum():
    """dbout is the column sum of dY over all rows of a slot (Y is affine in
    bout with unit slope); a planted transposition would break it."""
    rng = np.random.default_rng(4)
    PB, L, D, H = 5, 3, 4, 8
    dY = rng.normal(0, 1, (PB, L, D))
    g = F.backward_f64(rng.normal(0, 1, (PB, L, D)), params(rng, L, D, H), dY, 1e-5)
    np.testing.assert_allclose(g["bout"], dY.sum(axis=0), rtol=0, atol=1e-12)


def test_bit_array_entry_point_decodes_every_tensor():
    """ffn_slot_backward takes the storage formats (bf16 bits) of the
    forward's inputs and the upstream gradient: its gradients equal those of
    backward_f64 on the decoded values, key for key."""
    from synth import workloads as W
    case = W.FfnCase("tiny", B=2, T=4, D=8, k=2, P=2, affine=True, big_bias=True)
    inp = W.ffn_inputs(case)
    dy = W.ffn_upstream_grad(case)
    got = oracle.ffn_slot_backward(inp, dy, case.eps)
    q = {k: oracle.decode_bf16(inp[k]) for k in ("w1", "b1", "wout", "bout", "gx", "bx", "gg", "bg")}
    ref = F.backward_f64(oracle.decode_bf16(inp["x"]), q, oracle.decode_bf16(dy), case.eps)
    assert sorted(got) == sorted(ref) == sorted(["x", "w1", "b1", "wout", "bout", "gx", "bx", "gg", "bg"])
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k])
        assert got[k].shape == (inp[k].shape if k != "x" else inp["x"].shape)
