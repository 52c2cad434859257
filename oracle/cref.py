"""ctypes binding of the C++17 oracle (oracle/cpp/oracle.cpp) -- TEST
INFRASTRUCTURE ONLY, like the rest of this package.

The same operations as the numpy oracle (gemm.py, ffn.py, swiglu.py,
permute.py), written a second time in plain C++ with float64 sums and OpenMP
over output rows. The tests check one against the other; the benchmark times
this one as its CPU baseline. build() compiles it with g++ (no HIP, no GPU).
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "oracle.cpp")
LIB = os.path.join(HERE, "cpp", "liboracle.so")

_lib = None
_DT = {"bf16": 0, "e4m3": 1}
_LAYOUT = {"nk": 0, "kn": 1}


def build():
    """Compiles liboracle.so beside its source (g++ -O2 -fopenmp)."""
    tmp = f"{LIB}.{os.getpid()}.tmp"        # concurrent builders each write their own
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed on the C++ oracle:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def ensure_built():
    """Builds liboracle.so if it is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with oracle.cref.build()")
        _lib = ctypes.CDLL(LIB)
    return _lib


def _p(x):
    return x.ctypes.data_as(ctypes.c_void_p) if x is not None else None


def _arr(xs):
    xs = [np.ascontiguousarray(x) if x is not None else None for x in xs]
    ptrs = (ctypes.c_void_p * len(xs))(*[x.ctypes.data if x is not None else None for x in xs])
    return ptrs, xs


_i64, _d, _vp, _i = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int


def decode(bits, dtype):
    b = np.ascontiguousarray(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib().orc_decode(_p(b), _i(_DT[dtype]), _i64(b.size), _p(out))
    return out


def gemm_ag(a_slices, b, c, alpha, beta, rank, dtype="bf16", b_layout="nk", swiglu=False):
    P = len(a_slices)
    m, K = a_slices[0].shape
    b = np.ascontiguousarray(b)
    N = b.shape[0] if b_layout == "nk" else b.shape[1]
    n_out = N // 2 if swiglu else N
    c = np.ascontiguousarray(c) if (c is not None and beta != 0.0) else None
    ptrs, keep = _arr(a_slices)
    d = np.empty((P * m, n_out), dtype=np.float64)
    lib().orc_gemm_ag(ptrs, _i(P), _i(rank), _i64(m), _i64(N), _i64(K), _i(_DT[dtype]), _i(_LAYOUT[b_layout]),
                      _p(b), _p(c), _d(alpha), _d(beta), _i(1 if swiglu else 0), _p(d))
    return d


def gemm_rs(a, b, incoming, alpha, rank, P, b_layout="nk"):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    M, K = a.shape
    N = b.shape[0] if b_layout == "nk" else b.shape[1]
    ptrs, keep = _arr(incoming) if incoming is not None else (None, None)
    out = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_rs(_p(a), _i64(M), _i64(N), _i64(K), _i(P), _i(rank), _i(_LAYOUT[b_layout]), _p(b),
                      ptrs, _d(alpha), _p(out))
    return out


def gemm_ag_rotb(a, b_slices, c, alpha, beta, rank, dtype="bf16", b_layout="nk"):
    a = np.ascontiguousarray(a)
    M, K = a.shape
    P = len(b_slices)
    n = b_slices[0].shape[0] if b_layout == "nk" else b_slices[0].shape[1]
    c = np.ascontiguousarray(c) if (c is not None and beta != 0.0) else None
    ptrs, keep = _arr(b_slices)
    d = np.empty((M, P * n), dtype=np.float64)
    lib().orc_gemm_ag_rotb(_p(a), ptrs, _i(P), _i(rank), _i64(M), _i64(n), _i64(K), _i(_DT[dtype]),
                           _i(_LAYOUT[b_layout]), _p(c), _d(alpha), _d(beta), _p(d))
    return d


def gemm_rs_tileb(a, b, incoming, alpha, rank, P, b_layout="nk"):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    M, K = a.shape
    N = b.shape[0] if b_layout == "nk" else b.shape[1]
    ptrs, keep = _arr(incoming) if incoming is not None else (None, None)
    out = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_rs_tileb(_p(a), _i64(M), _i64(N), _i64(K), _i(P), _i(rank), _i(_LAYOUT[b_layout]), _p(b),
                            ptrs, _d(alpha), _p(out))
    return out


def ffn_slot_forward(inp, eps=1e-5):
    t = {k: np.ascontiguousarray(v) for k, v in inp.items()}
    PB, L, D = t["x"].shape
    H = t["wout"].shape[1]
    y = np.empty((PB, L, D), dtype=np.float64)
    lib().orc_ffn_slot_forward(_p(t["x"]), _i64(PB), _i64(L), _i64(D), _i64(H), _p(t["w1"]), _p(t["b1"]),
                               _p(t["wout"]), _p(t["bout"]), _p(t["gx"]), _p(t["bx"]), _p(t["gg"]),
                               _p(t["bg"]), _d(eps), _p(y))
    return y


def swiglu_hidden(x_shards, w13):
    P = len(x_shards)
    S, D = x_shards[0].shape
    w13 = np.ascontiguousarray(w13)
    F = w13.shape[1] // 2
    ptrs, keep = _arr(x_shards)
    h = np.empty((P * S, F), dtype=np.float64)
    lib().orc_swiglu_hidden(ptrs, _i(P), _i64(S), _i64(D), _i64(F), _p(w13), _p(h))
    return h


def dispatch(inputs, rank):
    P = len(inputs)
    B, T, D = inputs[0].shape
    ptrs, keep = _arr(inputs)
    out = np.empty((P * B, T // P, D), dtype=inputs[0].dtype)
    lib().orc_dispatch(ptrs, _i(P), _i(rank), _i64(B), _i64(T), _i64(D), _i(inputs[0].dtype.itemsize), _p(out))
    return out


def combine(ys, rank):
    P = len(ys)
    PB, L, D = ys[0].shape
    B = PB // P
    ptrs, keep = _arr(ys)
    out = np.empty((B, P * L, D), dtype=ys[0].dtype)
    lib().orc_combine(ptrs, _i(P), _i(rank), _i64(B), _i64(L), _i64(D), _i(ys[0].dtype.itemsize), _p(out))
    return out
