"""Staged all-gather GEMM and its reduce-scatter dual (test infrastructure only).

Operation ("Pytorch Op for blackwell distributed gemm", Usage and Note on
Tensor Layouts): D = alpha * (A @ B^T) + beta * C, A (M, K), B (N, K) row-major,
C and D (M, N). B may also be given (K, N) row-major (the weight layout of the
p04 FFN and of the torchtitan SwiGLU block), i.e. the matrix B^T itself.

All-gather form ("Distributed GEMM", Background, Figures 3-4; Approach,
schedule AllGather1D_TilingCD_RotatingA): A is split by rows into P slices
of m = M/P, slice s living on rank s. The local rank starts on its own slice
and the slices rotate, so stage t multiplies slice (rank + t) mod P and
writes rows [s*m, (s+1)*m) of D (C/D tiled by the same rows). The plain
reading adopted for "ring order" is this forward rotation; its mirror
(rank - t) gives the same D.

Reduce-scatter dual (Background, Figure 3; Approach, schedule
ReduceScatter1D_TilingA_RotatingC): A (M, K_shard) is this rank's K shard, so
E = alpha * A @ B^T is a partial sum. Its P row blocks are the partials
owed to the P ranks; stage t computes block (rank + 1 + t) mod P, the rank's
own block last. Blocks b != rank are emitted as is; the own block receives
the sum of the partials the other ranks computed for it (the rotating C),
added once, in full precision, before the single rounding of the output.

Column duals ("Distributed GEMM", Approach: the list of implemented
schedules names AllGather1D_TilingCD_RotatingB and
ReduceScatter1D_TilingB_RotatingC without spelling out their layout). The
reading adopted is the column dual of the two above. RotatingB: A (M, K) is
local and B's row slices (n = N/P rows each; in the (K, N) layout, column
blocks) rotate, so stage t multiplies slice (rank + t) mod P and writes
columns [s*n, (s+1)*n) of D. TilingB: the partial E = alpha * A @ B^T is
split into P column blocks owed to the P ranks; stage t computes block
(rank + 1 + t) mod P, the own block last, which adds the (M, n) partials
the other ranks computed for it.

Everything is float64; beta == 0 means C is not read (BLAS convention).
"""
import numpy as np

from .formats import decode, decode_bf16


def ag_stage_order(P, rank):
    """Slice index of each stage: local first, then the rotation."""
    return [(rank + t) % P for t in range(P)]


def rs_block_order(P, rank):
    """Output block of each reduce-scatter stage: own block last."""
    return [(rank + 1 + t) % P for t in range(P)]


def _b_as_nk(b, dtype, b_layout):
    Bm = decode(b, dtype)
    return Bm if b_layout == "nk" else Bm.T


def _swiglu_pairs(z):
    """silu(u) * v over the two column halves [u | v] of z."""
    n = z.shape[1] // 2
    u, v = z[:, :n], z[:, n:]
    return u / (1.0 + np.exp(-u)) * v


def gemm_ag(a_slices, b, c, alpha, beta, rank, dtype="bf16", b_layout="nk",
            swiglu=False, staged=True):
    """Full D (float64) of the all-gather form.

    staged=False computes the same product unstaged: the slices are first
    concatenated in rank order, then multiplied once.
    With swiglu, z = alpha * A @ B^T has N = 2n columns [u | v] and the
    output is silu(u) * v + beta * C with C (M, n).
    """
    P = len(a_slices)
    Bm = _b_as_nk(b, dtype, b_layout)
    m = a_slices[0].shape[0]
    n_out = Bm.shape[0] // 2 if swiglu else Bm.shape[0]
    Cm = decode_bf16(c) if beta != 0.0 else None

    def finish(z, rows):
        out = _swiglu_pairs(z) if swiglu else z
        if beta != 0.0:
            out = out + beta * Cm[rows]
        return out

    if not staged:
        A = np.concatenate([decode(s, dtype) for s in a_slices], axis=0)
        return finish(alpha * (A @ Bm.T), slice(0, P * m))

    D = np.empty((P * m, n_out), dtype=np.float64)
    for s in ag_stage_order(P, rank):
        rows = slice(s * m, (s + 1) * m)
        D[rows] = finish(alpha * (decode(a_slices[s], dtype) @ Bm.T), rows)
    return D


def gemm_ag_rows(a_slices, b, c, alpha, beta, dtype, b_layout, rows, swiglu=False):
    """Rows `rows` (global indices) of D, each from its own slice."""
    m = a_slices[0].shape[0]
    Bm = _b_as_nk(b, dtype, b_layout)
    A = np.stack([decode(a_slices[i // m][i % m], dtype) for i in rows])
    z = alpha * (A @ Bm.T)
    out = _swiglu_pairs(z) if swiglu else z
    if beta != 0.0:
        out = out + beta * decode_bf16(c[np.asarray(rows)])
    return out


def gemm_rs(a, b, incoming, alpha, rank, P, b_layout="nk"):
    """Full output (float64, M x N) of the reduce-scatter form.

    incoming[j] (j != rank) is the bf16 (m, N) partial of block `rank` that
    rank j computed; None entries (or incoming=None) contribute nothing.
    """
    Bm = _b_as_nk(b, "bf16", b_layout)
    A = decode_bf16(a)
    M = A.shape[0]
    m = M // P
    out = np.empty((M, Bm.shape[0]), dtype=np.float64)
    for blk in rs_block_order(P, rank):
        rows = slice(blk * m, (blk + 1) * m)
        part = alpha * (A[rows] @ Bm.T)
        if blk == rank and incoming is not None:
            for j in range(P):
                if j != rank and incoming[j] is not None:
                    part = part + decode_bf16(incoming[j])
        out[rows] = part
    return out


def gemm_rs_rows(a, b, incoming, alpha, rank, P, b_layout, rows):
    """Rows `rows` (global indices) of the reduce-scatter output."""
    Bm = _b_as_nk(b, "bf16", b_layout)
    A = decode_bf16(a[np.asarray(rows)])
    m = a.shape[0] // P
    out = alpha * (A @ Bm.T)
    for i, r in enumerate(rows):
        if r // m == rank and incoming is not None:
            for j in range(P):
                if j != rank and incoming[j] is not None:
                    out[i] = out[i] + decode_bf16(incoming[j][r % m])
    return out


def _slice_as_nk(x, dtype, b_layout):
    X = decode(x, dtype)
    return X if b_layout == "nk" else X.T


def gemm_ag_rotb(a, b_slices, c, alpha, beta, rank, dtype="bf16", b_layout="nk", staged=True):
    """Full D (float64, M x N) of the all-gather with rotating B.

    b_slices[s] is slice s of B: (n, K) rows of B, or in the (K, N) layout the
    (K, n) column block of B^T. staged=False concatenates the slices in rank
    order and multiplies once.
    """
    P = len(b_slices)
    A = decode(a, dtype)
    Bs = [_slice_as_nk(x, dtype, b_layout) for x in b_slices]
    n = Bs[0].shape[0]
    Cm = decode_bf16(c) if beta != 0.0 else None
    if not staged:
        out = alpha * (A @ np.concatenate(Bs, axis=0).T)
        return out + beta * Cm if beta != 0.0 else out
    D = np.empty((A.shape[0], P * n), dtype=np.float64)
    for s in ag_stage_order(P, rank):
        cols = slice(s * n, (s + 1) * n)
        part = alpha * (A @ Bs[s].T)
        D[:, cols] = part + beta * Cm[:, cols] if beta != 0.0 else part
    return D


def gemm_ag_rotb_rows(a, b_slices, c, alpha, beta, dtype, b_layout, rows):
    """Rows `rows` of the rotating-B all-gather output."""
    A = decode(a[np.asarray(rows)], dtype)
    B = np.concatenate([_slice_as_nk(x, dtype, b_layout) for x in b_slices], axis=0)
    out = alpha * (A @ B.T)
    if beta != 0.0:
        out = out + beta * decode_bf16(c[np.asarray(rows)])
    return out


def gemm_rs_tileb(a, b, incoming, alpha, rank, P, b_layout="nk"):
    """Full output (float64, M x N) of the reduce-scatter with tiled B.

    incoming[j] (j != rank) is the bf16 (M, n) partial of column block `rank`
    that rank j computed; None entries (or incoming=None) contribute nothing.
    """
    Bm = _b_as_nk(b, "bf16", b_layout)
    A = decode_bf16(a)
    n = Bm.shape[0] // P
    out = np.empty((A.shape[0], Bm.shape[0]), dtype=np.float64)
    for blk in rs_block_order(P, rank):
        cols = slice(blk * n, (blk + 1) * n)
        part = alpha * (A @ Bm[cols].T)
        if blk == rank and incoming is not None:
            for j in range(P):
                if j != rank and incoming[j] is not None:
                    part = part + decode_bf16(incoming[j])
        out[:, cols] = part
    return out


def gemm_rs_tileb_rows(a, b, incoming, alpha, rank, P, b_layout, rows):
    """Rows `rows` of the tiled-B reduce-scatter output."""
    Bm = _b_as_nk(b, "bf16", b_layout)
    A = decode_bf16(a[np.asarray(rows)])
    n = Bm.shape[0] // P
    out = alpha * (A @ Bm.T)
    if incoming is not None:
        cols = slice(rank * n, (rank + 1) * n)
        for j in range(P):
            if j != rank and incoming[j] is not None:
                out[:, cols] = out[:, cols] + decode_bf16(incoming[j][np.asarray(rows)])
    return out


def gemm_ag_multi(a_slices, bs, alpha, rank, dtype="bf16"):
    """Several column-parallel projections sharing one all-gathered input
    ("Add dist GEMM attention and FFN backend", Structure: AllGatherLinearMulti
    serves several linears that share one input, one all-gather for all;
    AllGatherFusedQKVLinear is the three-way case, wq / wk / wv in their own
    (N_i, K) layouts). Returns [alpha * A @ B_i^T for each B_i], A the slices
    gathered in rank order; stage t multiplies slice (rank + t) mod P by every
    B_i."""
    P = len(a_slices)
    m = a_slices[0].shape[0]
    outs = [np.empty((P * m, b.shape[0]), dtype=np.float64) for b in bs]
    Bs = [decode(b, dtype) for b in bs]
    for s in ag_stage_order(P, rank):
        As = decode(a_slices[s], dtype)
        for o, Bm in zip(outs, Bs):
            o[s * m:(s + 1) * m] = alpha * (As @ Bm.T)
    return outs
