"""Exact decoders of the storage formats (test infrastructure only).

bf16: the top 16 bits of an IEEE binary32 value.
OCP 8-bit E4M3FN ("float_e4m3" on the "Pytorch Op for blackwell distributed
gemm" page, Limitations): sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 holds subnormals M/8 * 2^-6; S.1111.111 is NaN; no
infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""
import numpy as np


def decode_bf16(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def decode_e4m3(bits):
    b = np.asarray(bits, dtype=np.uint8)
    sign = np.where(b >> 7, -1.0, 1.0)
    E = ((b >> 3) & 0xF).astype(np.int64)
    Mt = (b & 0x7).astype(np.float64)
    mag = np.where(E == 0, Mt / 8.0 * 2.0 ** -6, (1.0 + Mt / 8.0) * np.exp2(E - 7.0))
    out = sign * mag
    return np.where((b & 0x7F) == 0x7F, np.nan, out)


def decode(bits, dtype):
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "e4m3":
        return decode_e4m3(bits)
    raise ValueError(dtype)
