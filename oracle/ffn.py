"""Per-token-slot FFN, compute-only part (test infrastructure only).

From the p04 problem statement, "Computation and communication example" and
"Interface, layout, and parameters". For dispatched rows n in [0, P*B) and
slots l in [0, L), L = T/P, H = D*k:
  z       = X[n, l, :] @ w1[l] + b1[l]          w1 [L, D, 2H], b1 [L, 2H]
  (u, g)  = z[:H], z[H:]                          first half u, second half g
  LN(v)   = (v - mean v) / sqrt(mean (v - mean v)^2 + eps) * gamma + beta
  h       = LN_x(u) * silu(LN_gate(g))            norm_x / norm_gate: [H] each
  Y[n,l,:]= h @ wout[l] + bout[l]                 wout [L, H, D], bout [L, D]
with eps = 1e-5 and silu(t) = t * sigmoid(t) = t / (1 + e^-t). The population
variance is the one the statement prints (mean of squared deviations).
Everything is float64 with no intermediate rounding.
"""
import numpy as np

from .formats import decode_bf16


def silu(t):
    return t / (1.0 + np.exp(-t))


def layer_norm(v, gamma, beta, eps):
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    return (v - mu) / np.sqrt(var + eps) * gamma + beta


def _params(p):
    return {k: decode_bf16(p[k]) for k in ("w1", "b1", "wout", "bout", "gx", "bx", "gg", "bg")}


def _slot_rows(xrows, l, q, H, eps):
    z = xrows @ q["w1"][l] + q["b1"][l]
    u, g = z[:, :H], z[:, H:]
    h = layer_norm(u, q["gx"], q["bx"], eps) * silu(layer_norm(g, q["gg"], q["bg"], eps))
    return h @ q["wout"][l] + q["bout"][l]


def ffn_slot_forward(inp, eps=1e-5):
    """Y [P*B, L, D] (float64) from the dict of bf16 bit arrays `inp`
    (keys x, w1, b1, wout, bout, gx, bx, gg, bg)."""
    X = decode_bf16(inp["x"])
    q = _params(inp)
    PB, L, D = X.shape
    H = q["wout"].shape[1]
    Y = np.empty((PB, L, D), dtype=np.float64)
    for l in range(L):
        Y[:, l, :] = _slot_rows(X[:, l, :], l, q, H, eps)
    return Y


def ffn_slot_rows(inp, pairs, eps=1e-5):
    """Y[n, l, :] for each (n, l) in `pairs`, as an array [len(pairs), D]."""
    q = _params(inp)
    H = q["wout"].shape[1]
    out = []
    for n, l in pairs:
        xrow = decode_bf16(inp["x"][n, l])[None, :]
        out.append(_slot_rows(xrow, l, q, H, eps)[0])
    return np.stack(out)
