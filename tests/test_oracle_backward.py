"""Pins of the oracle's backward pass of the all-gather / reduce-scatter
linears (CPU).

The weight gradient is pinned against scalar brute force and, through the
adjoint identity, against the forward oracle: for Y = X W^T,
<dY, X E^T> = <dY^T X, E> for any E, and <dY, D W^T> = <dY W, D> for any D,
so a transposed operand, a dropped slice or a wrong stage row anywhere in
the gradient shows up as a mismatch with the forward product.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.backward import wgrad, wgrad_staged, wgrad_rows
from synth import gen


def bf16_bits(x):
    return gen.encode_bf16(np.asarray(x, dtype=np.float64))


def rand_bf16(rng, shape, lo=-2, hi=2):
    return bf16_bits(rng.integers(lo, hi + 1, size=shape))


def slices_of(a, P):
    m = a.shape[0] // P
    return [a[s * m:(s + 1) * m] for s in range(P)]


def test_wgrad_brute_force():
    rng = np.random.default_rng(0)
    M, N, K = 6, 3, 4
    g, x = rand_bf16(rng, (M, N)), rand_bf16(rng, (M, K))
    G, X = oracle.decode_bf16(g), oracle.decode_bf16(x)
    ref = np.zeros((N, K))
    for n, k, i in itertools.product(range(N), range(K), range(M)):
        ref[n, k] += G[i, n] * X[i, k]
    np.testing.assert_array_equal(wgrad(g, x), ref)
    np.testing.assert_array_equal(wgrad(g, x, alpha=-0.5), -0.5 * ref)


@pytest.mark.parametrize("P,rank,gathered", [(1, 0, "x"), (2, 1, "x"), (4, 2, "g"), (8, 5, "x"), (8, 0, "g")])
def test_staged_equals_unstaged_and_rows(P, rank, gathered):
    """Integer inputs: every partial sum is exact, so the staged sum (any
    rank, either gathered operand) equals the plain product exactly."""
    rng = np.random.default_rng(P * 10 + rank)
    m, N, K = 3, 5, 7
    g, x = rand_bf16(rng, (P * m, N)), rand_bf16(rng, (P * m, K))
    ref = wgrad(g, x, alpha=2.0)
    if gathered == "x":
        got = wgrad_staged(g, slices_of(x, P), "x", rank, alpha=2.0)
        rows = wgrad_rows(g, slices_of(x, P), "x", [4, 0, 2], alpha=2.0)
    else:
        got = wgrad_staged(x, slices_of(g, P), "g", rank, alpha=2.0)
        rows = wgrad_rows(x, slices_of(g, P), "g", [4, 0, 2], alpha=2.0)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(rows, ref[[4, 0, 2]])


def test_wgrad_is_the_adjoint_of_the_forward_in_w():
    """<dY, X E^T> computed by the forward oracle equals <dW, E>."""
    rng = np.random.default_rng(3)
    P, m, N, K = 4, 2, 3, 8
    x = rand_bf16(rng, (P * m, K))
    dy = rand_bf16(rng, (P * m, N))
    dW = wgrad_staged(dy, slices_of(x, P), "x", rank=1)
    for trial in range(3):
        e = rand_bf16(rng, (N, K))
        y = oracle.gemm_ag(slices_of(x, P), e, None, 1.0, 0.0, rank=2)
        assert np.sum(oracle.decode_bf16(dy) * y) == np.sum(dW * oracle.decode_bf16(e))


def test_dgrad_is_the_rs_dual_with_kn_weights():
    """dX_g = dY W: the reduce-scatter oracle with B = W read in the (K, N)
    layout gives it (no incoming partials), and <dY, D W^T> = <dY W, D>."""
    rng = np.random.default_rng(4)
    P, m, N, K = 4, 2, 3, 8
    w = rand_bf16(rng, (N, K))
    dy = rand_bf16(rng, (P * m, N))
    dxg = oracle.gemm_rs(dy, w, None, 1.0, rank=1, P=P, b_layout="kn")
    np.testing.assert_array_equal(dxg, oracle.decode_bf16(dy) @ oracle.decode_bf16(w))
    dd = rand_bf16(rng, (P * m, K))
    y = oracle.gemm_ag(slices_of(dd, P), w, None, 1.0, 0.0, rank=0)
    assert np.sum(oracle.decode_bf16(dy) * y) == np.sum(dxg * oracle.decode_bf16(dd))


def test_row_parallel_backward_forms():
    """LinearReduceScatter: dH = dOut_g W2 is the all-gather oracle with W2
    read in the (K, N) layout; dW2 = dOut_g^T H is the weight gradient with
    G gathered. Both against the adjoint of the forward Out = H W2^T."""
    rng = np.random.default_rng(5)
    P, m, D, F = 4, 2, 6, 5
    h = rand_bf16(rng, (P * m, F))
    w2 = rand_bf16(rng, (D, F))
    dout = rand_bf16(rng, (P * m, D))
    dh = oracle.gemm_ag(slices_of(dout, P), w2, None, 1.0, 0.0, rank=3, b_layout="kn")
    dw2 = wgrad_staged(h, slices_of(dout, P), "g", rank=3)
    out = oracle.decode_bf16(h) @ oracle.decode_bf16(w2).T
    np.testing.assert_array_equal(out, oracle.gemm_rs(h, w2, None, 1.0, rank=0, P=P))
    e_h, e_w = rand_bf16(rng, (P * m, F)), rand_bf16(rng, (D, F))
    dO = oracle.decode_bf16(dout)
    assert np.sum(dO * (oracle.decode_bf16(e_h) @ oracle.decode_bf16(w2).T)) == np.sum(dh * oracle.decode_bf16(e_h))
    assert np.sum(dO * (oracle.decode_bf16(h) @ oracle.decode_bf16(e_w).T)) == np.sum(dw2 * oracle.decode_bf16(e_w))


def test_wrong_stage_rows_would_be_caught():
    """A planted mistake (the local slice's G rows paired with the wrong X
    slice) changes the result: the staged pin above is sensitive to it."""
    rng = np.random.default_rng(6)
    P, m, N, K = 4, 3, 4, 5
    g, x = rand_bf16(rng, (P * m, N)), rand_bf16(rng, (P * m, K))
    xs = slices_of(x, P)
    wrong = [xs[(s + 1) % P] for s in range(P)]
    assert not np.array_equal(wgrad_staged(g, wrong, "x", 0), wgrad(g, x))
