"""SwiGLU tensor-parallel block share (test infrastructure only).

"Add dist GEMM attention and FFN backend" (torchtitan PR #4044), Structure:
AllGatherLinearMulti serves the SwiGLU pair w1/w3 with one all-gather of the
sequence shards; the FFN output projection w2 is the row-parallel
LinearReduceScatter. The gathered rows are the shards concatenated in rank
order (rows ordered (rank, batch, seq); batch 1 here). The SwiGLU itself is
silu(x @ w1) * (x @ w3), with w1 | w3 stored side by side as one (D, 2F)
column shard, w1 first; w2 is (F, D). The partial product h @ w2 is cut into
P row blocks, the reduce-scatter blocks.
"""
import numpy as np

from .formats import decode_bf16


def _silu(t):
    return t / (1.0 + np.exp(-t))


def swiglu_hidden(x_shards, w13):
    """h = silu(x @ w1) * (x @ w3), x = shards in rank order; float64 (M, F)."""
    x = np.concatenate([decode_bf16(s) for s in x_shards], axis=0)
    W = decode_bf16(w13)
    F = W.shape[1] // 2
    return _silu(x @ W[:, :F]) * (x @ W[:, F:])


def swiglu_hidden_rows(x_shards, w13, rows):
    S = x_shards[0].shape[0]
    x = np.stack([decode_bf16(x_shards[r // S][r % S]) for r in rows])
    W = decode_bf16(w13)
    F = W.shape[1] // 2
    return _silu(x @ W[:, :F]) * (x @ W[:, F:])


def swiglu_block(x_shards, w13, w2):
    """Partial output h @ w2 (float64, M x D), rows in P blocks of S."""
    return swiglu_hidden(x_shards, w13) @ decode_bf16(w2)
