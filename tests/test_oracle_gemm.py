"""Pins of the oracle's staged all-gather GEMM and reduce-scatter dual (CPU).

Each pin checks the oracle against something other than itself: scalar
brute force, closed forms, the unsharded product of the full matrices, or
mathematical invariants of the staging.
"""
import itertools

import numpy as np
import pytest

import oracle
from synth import gen


def bf16_bits(x):
    return gen.encode_bf16(np.asarray(x, dtype=np.float64))


def rand_int_bf16(rng, shape, lo=-2, hi=2):
    """Small integers: exactly representable, so every sum below is exact."""
    return bf16_bits(rng.integers(lo, hi + 1, size=shape))


def brute_ag(a_slices, b, c, alpha, beta, dec, b_layout):
    A = [[dec(v) for v in row] for s in a_slices for row in s]
    Bv = [[dec(v) for v in row] for row in b]
    M, K = len(A), len(A[0])
    N = len(Bv) if b_layout == "nk" else len(Bv[0])
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                bkj = Bv[j][k] if b_layout == "nk" else Bv[k][j]
                acc += A[i][k] * bkj
            cv = float(oracle.decode_bf16(c[i, j])) if beta != 0 else 0.0
            out[i][j] = alpha * acc + beta * cv
    return np.array(out)


@pytest.mark.parametrize("dtype,b_layout", [("bf16", "nk"), ("bf16", "kn"), ("e4m3", "nk")])
def test_ag_matches_brute_force(dtype, b_layout):
    rng = np.random.default_rng(1)
    P, m, N, K = 2, 3, 5, 8
    if dtype == "bf16":
        slices = [rand_int_bf16(rng, (m, K)) for _ in range(P)]
        b = rand_int_bf16(rng, (N, K) if b_layout == "nk" else (K, N))
        dec = lambda v: float(oracle.decode_bf16(v))
    else:
        slices = [gen.encode_e4m3(rng.integers(-4, 5, size=(m, K)) * 0.25) for _ in range(P)]
        b = gen.encode_e4m3(rng.integers(-4, 5, size=(N, K)) * 0.5)
        dec = lambda v: float(oracle.decode_e4m3(v))
    c = rand_int_bf16(rng, (P * m, N))
    for rank in range(P):
        got = oracle.gemm_ag(slices, b, c, 0.5, -2.0, rank, dtype, b_layout)
        ref = brute_ag(slices, b, c, 0.5, -2.0, dec, b_layout)
        assert np.array_equal(got, ref)


def test_ag_closed_form_ones():
    # A = B = 1  =>  D = alpha * K + beta * C
    P, m, N, K = 4, 8, 16, 512
    one = np.full((m, K), 0x3F80, np.uint16)
    b = np.full((N, K), 0x3F80, np.uint16)
    c = bf16_bits(np.random.default_rng(2).uniform(-1, 1, (P * m, N)))
    D = oracle.gemm_ag([one] * P, b, c, 1.0, 1.0, 0)
    assert np.array_equal(D, 512.0 + oracle.decode_bf16(c))


def test_ag_one_hot_selects_columns():
    rng = np.random.default_rng(3)
    P, m, K = 2, 5, 16
    perm = rng.permutation(K)[:7]
    b = np.zeros((7, K), np.uint16)
    b[np.arange(7), perm] = 0x3F80
    slices = [bf16_bits(rng.uniform(-1, 1, (m, K))) for _ in range(P)]
    D = oracle.gemm_ag(slices, b, None, 1.0, 0.0, 1)
    A = np.concatenate([oracle.decode_bf16(s) for s in slices])
    assert np.array_equal(D, A[:, perm])


def test_ag_beta_zero_never_reads_c_and_alpha_zero():
    rng = np.random.default_rng(4)
    slices = [bf16_bits(rng.uniform(-1, 1, (4, 8))) for _ in range(2)]
    b = bf16_bits(rng.uniform(-1, 1, (6, 8)))
    nan_c = np.full((8, 6), 0x7FC0, np.uint16)          # bf16 NaN
    assert np.isfinite(oracle.gemm_ag(slices, b, nan_c, 1.0, 0.0, 0)).all()
    c = bf16_bits(rng.uniform(-1, 1, (8, 6)))
    assert np.array_equal(oracle.gemm_ag(slices, b, c, 0.0, 1.5, 1), 1.5 * oracle.decode_bf16(c))


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_ag_staged_equals_unstaged_every_rank(P):
    rng = np.random.default_rng(5 + P)
    m, N, K = 3, 7, 24
    slices = [rand_int_bf16(rng, (m, K)) for _ in range(P)]
    b = rand_int_bf16(rng, (N, K))
    c = rand_int_bf16(rng, (P * m, N))
    ref = oracle.gemm_ag(slices, b, c, 1.0, 1.0, 0, staged=False)
    for rank in range(P):
        assert np.array_equal(oracle.gemm_ag(slices, b, c, 1.0, 1.0, rank), ref)


def test_ag_stage_order_is_a_rotation_local_first():
    for P in (1, 2, 4, 8):
        for r in range(P):
            order = oracle.ag_stage_order(P, r)
            assert order[0] == r and sorted(order) == list(range(P))
            assert all((order[t + 1] - order[t]) % P == 1 for t in range(P - 1))
            rs = oracle.rs_block_order(P, r)
            assert rs[-1] == r and sorted(rs) == list(range(P))


def test_ag_linearity_and_layouts():
    rng = np.random.default_rng(6)
    slices = [rand_int_bf16(rng, (4, 16)) for _ in range(2)]
    bnk = rand_int_bf16(rng, (6, 16))
    bkn = np.ascontiguousarray(bnk.T)
    c = rand_int_bf16(rng, (8, 6))
    d10 = oracle.gemm_ag(slices, bnk, None, 1.0, 0.0, 0)
    d = oracle.gemm_ag(slices, bkn, c, 0.5, 3.0, 1, b_layout="kn")
    assert np.array_equal(d, 0.5 * d10 + 3.0 * oracle.decode_bf16(c))


def test_ag_rows_sampling_matches_full():
    rng = np.random.default_rng(7)
    slices = [bf16_bits(rng.uniform(-1, 1, (5, 32))) for _ in range(4)]
    b = bf16_bits(rng.uniform(-1, 1, (9, 32)))
    c = bf16_bits(rng.uniform(-1, 1, (20, 9)))
    full = oracle.gemm_ag(slices, b, c, 1.0, 1.0, 2)
    rows = [0, 4, 5, 13, 19]
    np.testing.assert_allclose(oracle.gemm_ag_rows(slices, b, c, 1.0, 1.0, "bf16", "nk", rows),
                               full[rows], rtol=1e-13, atol=1e-13)


def test_ag_swiglu_pairs_halves():
    rng = np.random.default_rng(8)
    P, m, K, n = 2, 3, 8, 4
    slices = [rand_int_bf16(rng, (m, K), -1, 1) for _ in range(P)]
    w = rand_int_bf16(rng, (K, 2 * n), -1, 1)
    got = oracle.gemm_ag(slices, w, None, 1.0, 0.0, 0, b_layout="kn", swiglu=True)
    A = np.concatenate([oracle.decode_bf16(s) for s in slices])
    W = oracle.decode_bf16(w)
    for i, j in itertools.product(range(P * m), range(n)):
        u = sum(A[i, k] * W[k, j] for k in range(K))
        v = sum(A[i, k] * W[k, n + j] for k in range(K))
        assert abs(got[i, j] - u / (1 + np.exp(-u)) * v) < 1e-12


@pytest.mark.parametrize("P", [2, 4, 8])
def test_rs_distributed_identity(P):
    """Simulate all P ranks: rank r holds K-shard r of A and B. Feeding every
    rank the partials its peers emitted for its block must give the rows of
    the unsharded product A_full @ B_full^T (integer data: exact)."""
    rng = np.random.default_rng(10 + P)
    m, N, Ks = 3, 5, 4
    A = [rand_int_bf16(rng, (P * m, Ks), -1, 1) for _ in range(P)]
    Bs = [rand_int_bf16(rng, (N, Ks), -1, 1) for _ in range(P)]
    emitted = [oracle.gemm_rs(A[r], Bs[r], None, 1.0, r, P) for r in range(P)]
    full = np.concatenate([oracle.decode_bf16(a) for a in A], axis=1) @ \
        np.concatenate([oracle.decode_bf16(b) for b in Bs], axis=1).T
    for r in range(P):
        incoming = [None if j == r else bf16_bits(emitted[j][r * m:(r + 1) * m]) for j in range(P)]
        out = oracle.gemm_rs(A[r], Bs[r], incoming, 1.0, r, P)
        assert np.array_equal(out[r * m:(r + 1) * m], full[r * m:(r + 1) * m])
        for blk in range(P):       # emitted blocks are this rank's own partials
            if blk != r:
                own = oracle.decode_bf16(A[r][blk * m:(blk + 1) * m]) @ oracle.decode_bf16(Bs[r]).T
                assert np.array_equal(out[blk * m:(blk + 1) * m], own)


def test_rs_rows_and_layout():
    rng = np.random.default_rng(20)
    P, m, N, K = 4, 3, 6, 8
    a = bf16_bits(rng.uniform(-1, 1, (P * m, K)))
    bnk = bf16_bits(rng.uniform(-1, 1, (N, K)))
    inc = [None if j == 1 else bf16_bits(rng.uniform(-1, 1, (m, N))) for j in range(P)]
    full = oracle.gemm_rs(a, bnk, inc, 0.5, 1, P)
    full_kn = oracle.gemm_rs(a, np.ascontiguousarray(bnk.T), inc, 0.5, 1, P, b_layout="kn")
    np.testing.assert_array_equal(full, full_kn)
    rows = [0, 3, 4, 5, 11]
    np.testing.assert_allclose(oracle.gemm_rs_rows(a, bnk, inc, 0.5, 1, P, "nk", rows), full[rows],
                               rtol=1e-13, atol=1e-13)


# ---- column duals: rotating B (all-gather) and tiled B (reduce-scatter)

def col_blocks(b_nk, P, b_layout):
    """B (N, K) split into P row slices, in the layout the call takes."""
    n = b_nk.shape[0] // P
    sl = [b_nk[s * n:(s + 1) * n] for s in range(P)]
    return sl if b_layout == "nk" else [np.ascontiguousarray(x.T) for x in sl]


@pytest.mark.parametrize("dtype,b_layout", [("bf16", "nk"), ("bf16", "kn"), ("e4m3", "nk")])
def test_ag_rotb_matches_brute_force(dtype, b_layout):
    """Integer data: the staged column blocks equal a plain triple loop."""
    rng = np.random.default_rng(31)
    P, M, n, K = 3, 4, 2, 8
    if dtype == "bf16":
        a = rand_int_bf16(rng, (M, K))
        b = rand_int_bf16(rng, (P * n, K))
        dec = lambda v: float(oracle.decode_bf16(v))
    else:
        a = gen.encode_e4m3(rng.integers(-4, 5, size=(M, K)) * 0.25)
        b = gen.encode_e4m3(rng.integers(-4, 5, size=(P * n, K)) * 0.5)
        dec = lambda v: float(oracle.decode_e4m3(v))
    c = rand_int_bf16(rng, (M, P * n))
    ref = brute_ag([a], b, c, 0.5, -2.0, dec, "nk")
    for rank in range(P):
        got = oracle.gemm_ag_rotb(a, col_blocks(b, P, b_layout), c, 0.5, -2.0, rank, dtype, b_layout)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("P", [2, 4, 8])
def test_ag_rotb_is_the_transposed_rota(P):
    """(A B^T)^T = B A^T: rotating B over B's row slices is the rotating-A
    all-gather with the roles of A and B exchanged, transposed."""
    rng = np.random.default_rng(40 + P)
    M, n, K = 5, 3, 16
    a = bf16_bits(rng.uniform(-1, 1, (M, K)))
    b = bf16_bits(rng.uniform(-1, 1, (P * n, K)))
    c = bf16_bits(rng.uniform(-1, 1, (M, P * n)))
    for rank in (0, P - 1):
        got = oracle.gemm_ag_rotb(a, col_blocks(b, P, "nk"), c, 0.75, 0.5, rank)
        dual = oracle.gemm_ag(col_blocks(b, P, "nk"), a, np.ascontiguousarray(c.T), 0.75, 0.5, rank)
        np.testing.assert_allclose(got, dual.T, rtol=1e-13, atol=1e-13)
        unst = oracle.gemm_ag_rotb(a, col_blocks(b, P, "kn"), c, 0.75, 0.5, rank, b_layout="kn", staged=False)
        np.testing.assert_allclose(got, unst, rtol=1e-13, atol=1e-13)
    rows = [0, 2, 4]
    np.testing.assert_allclose(oracle.gemm_ag_rotb_rows(a, col_blocks(b, P, "nk"), c, 0.75, 0.5, "bf16", "nk",
                                                        rows), got[rows], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("P", [2, 4, 8])
def test_rs_tileb_is_the_transposed_rs(P):
    """(A B^T)^T = B A^T: the tiled-B reduce-scatter over B's row blocks is
    the tiled-A reduce-scatter with A and B exchanged, transposed, and the
    incoming (M, n) partials transposed to (n, M)."""
    rng = np.random.default_rng(60 + P)
    M, n, K = 4, 3, 8
    a = bf16_bits(rng.uniform(-1, 1, (M, K)))
    b = bf16_bits(rng.uniform(-1, 1, (P * n, K)))
    for rank in (0, P // 2):
        inc = [None if j == rank else bf16_bits(rng.uniform(-1, 1, (M, n))) for j in range(P)]
        got = oracle.gemm_rs_tileb(a, b, inc, 0.5, rank, P)
        inc_t = [None if x is None else np.ascontiguousarray(x.T) for x in inc]
        dual = oracle.gemm_rs(b, a, inc_t, 0.5, rank, P)
        np.testing.assert_allclose(got, dual.T, rtol=1e-13, atol=1e-13)
        got_kn = oracle.gemm_rs_tileb(a, np.ascontiguousarray(b.T), inc, 0.5, rank, P, b_layout="kn")
        np.testing.assert_array_equal(got, got_kn)
        rows = [0, 1, 3]
        np.testing.assert_allclose(oracle.gemm_rs_tileb_rows(a, b, inc, 0.5, rank, P, "nk", rows), got[rows],
                                   rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("P", [2, 4])
def test_rs_tileb_distributed_identity(P):
    """Simulate all P ranks: rank r holds K-shard r of A and B. Feeding every
    rank the column partials its peers emitted for its block gives the
    columns of the unsharded product (integer data: exact)."""
    rng = np.random.default_rng(80 + P)
    M, n, Ks = 3, 2, 4
    A = [rand_int_bf16(rng, (M, Ks), -1, 1) for _ in range(P)]
    Bs = [rand_int_bf16(rng, (P * n, Ks), -1, 1) for _ in range(P)]
    emitted = [oracle.gemm_rs_tileb(A[r], Bs[r], None, 1.0, r, P) for r in range(P)]
    full = np.concatenate([oracle.decode_bf16(a) for a in A], axis=1) @ \
        np.concatenate([oracle.decode_bf16(b) for b in Bs], axis=1).T
    for r in range(P):
        incoming = [None if j == r else bf16_bits(emitted[j][:, r * n:(r + 1) * n]) for j in range(P)]
        out = oracle.gemm_rs_tileb(A[r], Bs[r], incoming, 1.0, r, P)
        assert np.array_equal(out[:, r * n:(r + 1) * n], full[:, r * n:(r + 1) * n])


def test_ag_multi_brute_force_and_concatenation():
    """Several projections of one gathered input: brute force on a tiny case,
    and the concatenation identity [A Bq^T | A Bk^T | A Bv^T] = A [Bq; Bk; Bv]^T
    against the single-B all-gather oracle."""
    rng = np.random.default_rng(21)
    P, m, K = 2, 2, 3
    slices = [rand_int_bf16(rng, (m, K)) for _ in range(P)]
    bs = [rand_int_bf16(rng, (n, K)) for n in (3, 1, 2)]
    outs = oracle.gemm_ag_multi(slices, bs, 0.5, rank=1)
    A = [[oracle.decode_bf16(v) for v in row] for s in slices for row in s]
    for o, b in zip(outs, bs):
        for i in range(P * m):
            for j in range(b.shape[0]):
                ref = 0.5 * sum(A[i][k] * oracle.decode_bf16(b[j, k]) for k in range(K))
                assert o[i, j] == ref
    rng = np.random.default_rng(22)
    P, m, K = 4, 3, 16
    slices = [rand_int_bf16(rng, (m, K)) for _ in range(P)]
    bs = [rand_int_bf16(rng, (n, K)) for n in (8, 4, 4)]
    outs = oracle.gemm_ag_multi(slices, bs, 1.0, rank=2, dtype="bf16")
    whole = oracle.gemm_ag(slices, np.concatenate(bs, axis=0), None, 1.0, 0.0, rank=0)
    np.testing.assert_array_equal(np.concatenate(outs, axis=1), whole)


# ---- reduce-scatter with alpha != 1 and incoming partials: alpha scales the
# own partial product only; the incoming partials are added as they arrive

def brute_rs(a, b, incoming, alpha, rank, P, tile_b):
    """Scalar loops over the definition: out = alpha * A B^T everywhere, plus,
    on the own block (rows of block `rank`, or columns with tile_b), the sum
    of the peers' bf16 partials, unscaled."""
    A = oracle.decode_bf16(a)
    Bv = oracle.decode_bf16(b)
    M, K = A.shape
    N = Bv.shape[0]
    m, n = M // P, N // P
    out = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(A[i, k]) * float(Bv[j, k])
            v = alpha * acc
            own = (j // n == rank) if tile_b else (i // m == rank)
            if own:
                for src in range(P):
                    if src != rank and incoming[src] is not None:
                        x = incoming[src][i, j - rank * n] if tile_b else incoming[src][i - rank * m, j]
                        v += float(oracle.decode_bf16(x))
            out[i, j] = v
    return out


@pytest.mark.parametrize("tile_b", [False, True])
@pytest.mark.parametrize("P,rank", [(2, 1), (4, 2)])
def test_rs_alpha_scales_own_partial_only(tile_b, P, rank):
    """Integer data, alpha = 0.75: every sum is exact, so the oracle must
    equal the scalar brute force bit for bit. Scaling the incoming partials
    by alpha as well (a plausible mistake) moves the own block by
    0.25 * sum(incoming), which is nonzero here."""
    rng = np.random.default_rng(90 + P + 10 * tile_b)
    m, n, K = 3, 2, 8
    M, N = P * m, P * n
    a = rand_int_bf16(rng, (M, K))
    b = rand_int_bf16(rng, (N, K))
    shape = (M, n) if tile_b else (m, N)
    inc = [None if j == rank else rand_int_bf16(rng, shape, -3, 3) for j in range(P)]
    assert any(np.any(oracle.decode_bf16(x) != 0) for x in inc if x is not None)
    ref = brute_rs(a, b, inc, 0.75, rank, P, tile_b)
    got = (oracle.gemm_rs_tileb if tile_b else oracle.gemm_rs)(a, b, inc, 0.75, rank, P)
    assert np.array_equal(got, ref)
    got_kn = (oracle.gemm_rs_tileb if tile_b else oracle.gemm_rs)(a, np.ascontiguousarray(b.T), inc, 0.75,
                                                                  rank, P, b_layout="kn")
    assert np.array_equal(got_kn, ref)


@pytest.mark.parametrize("tile_b", [False, True])
@pytest.mark.parametrize("P", [2, 4])
def test_rs_distributed_identity_with_alpha(tile_b, P):
    """Every rank runs with the same alpha and feeds on the partials its
    peers emitted (already scaled by alpha): the own block must then be
    alpha times the unsharded product, exactly (integer data, alpha = 0.75,
    |partials| <= 16, so alpha * E is exact in bf16)."""
    rng = np.random.default_rng(120 + P + 10 * tile_b)
    m, n, Ks = 3, 2, 4
    M, N = P * m, P * n
    alpha = 0.75
    A = [rand_int_bf16(rng, (M, Ks), -1, 1) for _ in range(P)]
    Bs = [rand_int_bf16(rng, (N, Ks), -1, 1) for _ in range(P)]
    fn = oracle.gemm_rs_tileb if tile_b else oracle.gemm_rs
    emitted = [fn(A[r], Bs[r], None, alpha, r, P) for r in range(P)]
    full = np.concatenate([oracle.decode_bf16(x) for x in A], axis=1) @ \
        np.concatenate([oracle.decode_bf16(x) for x in Bs], axis=1).T
    for r in range(P):
        if tile_b:
            blk = (slice(None), slice(r * n, (r + 1) * n))
        else:
            blk = (slice(r * m, (r + 1) * m), slice(None))
        incoming = [None if j == r else bf16_bits(emitted[j][blk]) for j in range(P)]
        out = fn(A[r], Bs[r], incoming, alpha, r, P)
        assert np.array_equal(out[blk], alpha * full[blk])


@pytest.mark.parametrize("tile_b", [False, True])
def test_rs_planted_alpha_on_incoming_is_caught(tile_b):
    """A copy of the reduce-scatter oracle that also scales the incoming
    partials by alpha differs from the brute force: the alpha pins above can
    fail."""
    rng = np.random.default_rng(150 + tile_b)
    P, rank, m, n, K = 4, 1, 3, 2, 8
    a = rand_int_bf16(rng, (P * m, K))
    b = rand_int_bf16(rng, (P * n, K))
    shape = (P * m, n) if tile_b else (m, P * n)
    inc = [None if j == rank else rand_int_bf16(rng, shape, -3, 3) for j in range(P)]
    fn = oracle.gemm_rs_tileb if tile_b else oracle.gemm_rs
    bad = fn(a, b, None, 0.75, rank, P)
    blk = (slice(None), slice(rank * n, (rank + 1) * n)) if tile_b else (slice(rank * m, (rank + 1) * m), slice(None))
    bad[blk] += 0.75 * sum(oracle.decode_bf16(x) for x in inc if x is not None)
    assert not np.array_equal(bad, brute_rs(a, b, inc, 0.75, rank, P, tile_b))
