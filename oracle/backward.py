"""Backward pass of the all-gather and reduce-scatter linears (test
infrastructure only).

Source: "Add dist GEMM attention and FFN backend" (torchtitan PR #4044),
Structure. AllGatherLinear (column-parallel: all-gather the sequence shard,
then GEMM) and LinearReduceScatter (row-parallel: GEMM, then reduce-scatter)
are autograd Functions whose backward needs the same two collectives, an
all-gather and a reduce-scatter.

Reading adopted (the page names the Functions, not their gradients; these
are the gradients of the two products):
  * AllGatherLinear, Y = X_g W^T with X_g the rank-ordered gathered rows and
    W (N_loc, K) this rank's weight shard in the (out, in) layout:
      dX_g = dY W, a partial over the ranks' N shards, so this rank's dX is a
      reduce-scatter: the RS dual with B = W read in the (K, N) layout;
      dW = dY^T X_g, a contraction over the gathered token rows.
  * LinearReduceScatter, Out = H W2^T reduce-scattered, W2 (D, F_loc):
      dH = dOut_g W2, an all-gather GEMM with B = W2 in the (K, N) layout;
      dW2 = dOut_g^T H, a contraction over the gathered token rows.
The weight gradient is therefore one form for both Functions:
      out (N, K) = alpha * sum_i G[i, n] X[i, k],   G (M, N), X (M, K),
with the M token rows split into P slices of m = M/P and one of the two
operands arriving as those slices (the all-gathered one). Staging follows
the all-gather form ("Distributed GEMM", Background, Figures 3-4): stage t
contributes the rows of slice (rank + t) mod P, local first. Staging splits
the contraction, so every stage adds into the same output; the staged sum
equals the unstaged product up to rounding order.

Everything is float64 on decoded bf16 inputs.
"""
import numpy as np

from .formats import decode_bf16
from .gemm import ag_stage_order


def wgrad(g, x, alpha=1.0):
    """out (N, K) = alpha * G^T X: the plain definition."""
    return alpha * (decode_bf16(g).T @ decode_bf16(x))


def wgrad_staged(local, slices, gathered, rank, alpha=1.0):
    """The staged weight gradient.

    gathered = "x": `local` is G (M, N) and `slices` the P row slices of X.
    gathered = "g": `local` is X (M, K) and `slices` the P row slices of G.
    Stage t adds the contribution of slice s = (rank + t) mod P: the rows
    [s*m, (s+1)*m) of both operands.
    """
    P = len(slices)
    m = slices[0].shape[0]
    L = decode_bf16(local)
    out = None
    for s in ag_stage_order(P, rank):
        rows = slice(s * m, (s + 1) * m)
        S = decode_bf16(slices[s])
        part = L[rows].T @ S if gathered == "x" else S.T @ L[rows]
        out = part if out is None else out + part
    return alpha * out


def wgrad_rows(local, slices, gathered, rows, alpha=1.0):
    """Rows `rows` (indices n of the output) of the weight gradient."""
    rows = np.asarray(rows)
    if gathered == "x":
        G = decode_bf16(local)[:, rows]
        X = np.concatenate([decode_bf16(s) for s in slices], axis=0)
    else:
        G = np.concatenate([decode_bf16(s) for s in slices], axis=0)[:, rows]
        X = decode_bf16(local)
    return alpha * (G.T @ X)
