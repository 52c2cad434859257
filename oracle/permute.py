"""All-to-All dispatch and combine as layout maps (test infrastructure only).

p04 problem statement, "Interface, layout, and parameters" and "Computation
and communication example":
  dispatch = A2A(inputs, split_dim=1, concat_dim=0): every rank s cuts its
    [B, T, D] input along T into P slices of L = T/P tokens and sends slice r
    to rank r, which concatenates what it receives along the batch dimension
    in source-rank order: out_r[s*B + b, l, :] = in_s[b, r*L + l, :].
  combine = A2A(Y, split_dim=0, concat_dim=1): rank s cuts its [P*B, L, D]
    output along the first dimension into P slices of B and sends slice r to
    rank r, which concatenates along tokens in source-rank order:
    out_r[b, s*L + l, :] = Y_s[r*B + b, l, :].
A single GPU holds all P ranks' buffers, so both are pure permutations and
exactly one result is correct. Works on any element type (raw bits).
"""
import numpy as np


def dispatch(inputs, rank):
    P = len(inputs)
    B, T, D = inputs[0].shape
    assert T % P == 0, "the statement requires T % P == 0"
    L = T // P
    out = np.empty((P * B, L, D), dtype=inputs[0].dtype)
    for s in range(P):
        out[s * B:(s + 1) * B] = inputs[s][:, rank * L:(rank + 1) * L, :]
    return out


def combine(ys, rank):
    P = len(ys)
    PB, L, D = ys[0].shape
    B = PB // P
    out = np.empty((B, P * L, D), dtype=ys[0].dtype)
    for s in range(P):
        out[:, s * L:(s + 1) * L, :] = ys[s][rank * B:(rank + 1) * B]
    return out
