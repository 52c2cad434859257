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
    # e^-t overflows to inf for t below about -709; t / inf is then the exact
    # limit -0.0, so the overflow warning is silenced, not the value changed
    with np.errstate(over="ignore"):
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


# ---------------------------------------------------------------------------
# Backward. The p04 statement ("Interface, layout, and parameters") asks that
# autograd propagate through the layer to its input and every parameter; the
# gradients below are those of the forward above, written out by hand:
#   dwout[l] = h^T dY,  dbout[l] = sum_n dY,  dh = dY wout[l]^T
#   da = dh * silu(b),  db = dh * a * silu'(b),  silu'(t) = s(t)(1 + t(1 - s(t)))
#     with a = LN_x(u), b = LN_gate(g), s the logistic function
#   dgx += sum_n da * xhat_u,  dbx += sum_n da,  (gate likewise with xhat_g, db)
#   du = (dxh - mean(dxh) - xhat_u * mean(dxh * xhat_u)) / sqrt(var_u + eps),
#     dxh = da * gx  (the LayerNorm backward; g likewise)
#   dz = [du | dg],  dw1[l] = X^T dz,  db1[l] = sum_n dz,  dX = dz w1[l]^T
# gamma / beta are shared by all slots, so their gradients sum over slots.
# ---------------------------------------------------------------------------
def forward_f64(X, q, eps):
    """The forward on float64 arrays (X [PB, L, D]; q the decoded parameters);
    used by the finite-difference pins of the backward."""
    PB, L, D = X.shape
    H = q["wout"].shape[1]
    Y = np.empty((PB, L, D), dtype=np.float64)
    for l in range(L):
        Y[:, l, :] = _slot_rows(X[:, l, :], l, q, H, eps)
    return Y


def _ln_parts(v, eps):
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    return (v - mu) * r, r


def _ln_backward(dxh, xhat, r):
    return (dxh - dxh.mean(axis=-1, keepdims=True) - xhat * (dxh * xhat).mean(axis=-1, keepdims=True)) * r


def backward_f64(X, q, dY, eps):
    """Gradients (float64) of L = sum(dY * Y) for the forward_f64 layer."""
    PB, L, D = X.shape
    H = q["wout"].shape[1]
    g = {k: np.zeros_like(q[k]) for k in ("w1", "b1", "wout", "bout", "gx", "bx", "gg", "bg")}
    dX = np.empty_like(X)
    for l in range(L):
        Xl, dYl = X[:, l, :], dY[:, l, :]
        z = Xl @ q["w1"][l] + q["b1"][l]
        u, gt = z[:, :H], z[:, H:]
        xu, ru = _ln_parts(u, eps)
        xg, rg = _ln_parts(gt, eps)
        a = xu * q["gx"] + q["bx"]
        b = xg * q["gg"] + q["bg"]
        sg = 1.0 / (1.0 + np.exp(-b))
        s = b * sg
        h = a * s
        g["wout"][l] = h.T @ dYl
        g["bout"][l] = dYl.sum(axis=0)
        dh = dYl @ q["wout"][l].T
        da = dh * s
        db = dh * a * sg * (1.0 + b * (1.0 - sg))
        g["gx"] += (da * xu).sum(axis=0)
        g["bx"] += da.sum(axis=0)
        g["gg"] += (db * xg).sum(axis=0)
        g["bg"] += db.sum(axis=0)
        dz = np.concatenate([_ln_backward(da * q["gx"], xu, ru), _ln_backward(db * q["gg"], xg, rg)], axis=1)
        g["w1"][l] = Xl.T @ dz
        g["b1"][l] = dz.sum(axis=0)
        dX[:, l, :] = dz @ q["w1"][l].T
    g["x"] = dX
    return g


def ffn_slot_backward(inp, dy, eps=1e-5):
    """Gradients (float64) of the layer for the bf16 bit arrays `inp` (the
    forward's keys) and the upstream gradient `dy` [P*B, L, D] (bf16 bits):
    dict with keys x, w1, b1, wout, bout, gx, bx, gg, bg."""
    return backward_f64(decode_bf16(inp["x"]), _params(inp), decode_bf16(dy), eps)
