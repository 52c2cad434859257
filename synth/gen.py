"""Counter-based random streams and storage-format encoders.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014). Output i of the stream with key k is
mix(k + (i + 1) * GAMMA), so any element can be drawn without the ones before
it, and chunked generation is exact.

Normals: the Box-Muller transform (Box and Muller, 1958). Element 2p takes the
cosine branch and element 2p + 1 the sine branch of pair p, which consumes
counters 2p and 2p + 1.

Encoders: round-to-nearest, ties-to-even, to bf16 (8 significant bits) and to
OCP 8-bit E4M3FN (bias 7, 3 mantissa bits, subnormal quantum 2^-9, largest
finite value 448, no infinities), saturating at +-448.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _fnv1a64(text):
    h = 0xCBF29CE484222325
    for ch in text.encode():
        h = ((h ^ ch) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return np.uint64(h)


def stream_key(seed, tag):
    """Key of the stream named `tag` under integer `seed`."""
    with np.errstate(over="ignore"):
        base = _mix(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + GAMMA)
    return np.uint64(_mix(base ^ _fnv1a64(tag)))


def _raw(key, start, count):
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + (idx + np.uint64(1)) * GAMMA)


def _u01(key, start, count):
    # 53 high bits -> double in [0, 1)
    return (_raw(key, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _chunked(n, fill):
    """Runs fill(start, count) over _CHUNK-sized pieces on a thread pool.
    Every element depends only on its own counter, so the pieces are
    independent and the result does not depend on the thread count."""
    starts = list(range(0, n, _CHUNK))
    if len(starts) <= 1:
        for s in starts:
            fill(s, min(_CHUNK, n - s))
        return
    workers = min(len(starts), int(os.environ.get("SYNTH_THREADS", os.cpu_count() or 1)), 16)
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(lambda s: fill(s, min(_CHUNK, n - s)), starts))


def uniform(key, n, lo, hi):
    """n doubles, U[lo, hi)."""
    out = np.empty(n, dtype=np.float64)

    def fill(s, c):
        out[s:s + c] = lo + (hi - lo) * _u01(key, s, c)
    _chunked(n, fill)
    return out


def normal(key, n, mean=0.0, std=1.0):
    """n doubles, N(mean, std^2), by Box-Muller over counter pairs."""
    out = np.empty(n, dtype=np.float64)

    def fill(s, c):                    # _CHUNK is even, so pairs never straddle
        first, last = s // 2, (s + c - 1) // 2
        npair = last - first + 1
        u = _u01(key, 2 * first, 2 * npair).reshape(npair, 2)
        r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))       # 1 - u in (0, 1]
        th = 2.0 * np.pi * u[:, 1]
        pair = np.stack([r * np.cos(th), r * np.sin(th)], axis=1).reshape(-1)
        off = s - 2 * first
        out[s:s + c] = mean + std * pair[off:off + c]
    _chunked(n, fill)
    return out


def encode_bf16(x):
    """float64 array -> uint16 bf16 bit patterns, round-to-nearest-even.

    Values are rounded directly from float64 to 8 significant bits (no double
    rounding through float32); the result is exact in float32, whose top 16
    bits are the bf16 pattern. Intended for finite values in the bf16 normal
    range or zero.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def encode_e4m3(x):
    """float64 array -> uint8 OCP E4M3FN bit patterns, RNE, saturating to +-448."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qexp = np.maximum(e - 4, -9)             # 4 significant bits; subnormal quantum 2^-9
    q = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)
    q = np.clip(q, -448.0, 448.0)
    a = np.abs(q)
    sign = (np.signbit(q)).astype(np.uint8) << np.uint8(7)
    normal_ = a >= 2.0 ** -6
    _, ea = np.frexp(np.where(normal_, a, 1.0))
    E = np.where(normal_, ea - 1 + 7, 0)     # a = (1 + M/8) * 2^(E-7)
    M = np.where(normal_, np.ldexp(a, -(ea - 1)) * 8 - 8, a * 512.0)
    return (sign | (E.astype(np.uint8) << np.uint8(3)) | M.astype(np.uint8)).astype(np.uint8)


def _encode_chunked(v, enc, dtype):
    out = np.empty(v.shape[0], dtype=dtype)

    def fill(s, c):
        out[s:s + c] = enc(v[s:s + c])
    _chunked(v.shape[0], fill)
    return out


def uniform_bf16(key, shape, lo, hi):
    n = int(np.prod(shape))
    return _encode_chunked(uniform(key, n, lo, hi), encode_bf16, np.uint16).reshape(shape)


def normal_bf16(key, shape, mean=0.0, std=1.0):
    n = int(np.prod(shape))
    return _encode_chunked(normal(key, n, mean, std), encode_bf16, np.uint16).reshape(shape)


def normal_e4m3(key, shape, scale=1.0, clip=448.0):
    n = int(np.prod(shape))
    v = np.clip(scale * normal(key, n), -clip, clip)
    return _encode_chunked(v, encode_e4m3, np.uint8).reshape(shape)


def small_ints(key, n, lo, hi):
    """n integers drawn uniformly from [lo, hi] (floor of a uniform draw)."""
    return np.floor(uniform(key, n, lo, hi + 1)).astype(np.int64)


def shifted_rows(key, rows, cols, lo, hi, encode, dtype, step=37):
    """(rows, cols) storage codes whose row r is one seeded sequence of small
    integers in [lo, hi], cyclically shifted by r * step places, and encoded
    with `encode` (exact for small integers). Cheap at any size: only the one
    sequence (2 * cols + 1 values) is drawn; every row is a copy of a window
    of it, so tensors of several GiB are built by memory copies alone."""
    period = 2 * cols + 1
    seq = encode(small_ints(key, period, lo, hi).astype(np.float64)).astype(dtype)
    windows = np.lib.stride_tricks.sliding_window_view(np.concatenate([seq, seq]), cols)
    return windows[(np.arange(rows, dtype=np.int64) * step) % period]
