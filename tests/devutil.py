"""Device helpers for the GPU tests: move raw bit arrays to and from the GPU."""
import sys

import numpy as np
import torch


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def dev(bits):
    """numpy uint16 (bf16 bits) / uint8 (e4m3 bits) -> contiguous cuda tensor of the same bits."""
    if bits is None:
        return None
    if bits.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    if bits.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    raise TypeError(bits.dtype)


def bf16_empty(*shape, fill_nan=True):
    t = torch.empty(*shape, dtype=torch.int16, device="cuda")
    if fill_nan:
        t.fill_(0x7FC0)            # bf16 quiet NaN: any element left unwritten fails parity
    return t


def host_f64(t):
    """bf16 bits on the GPU -> float64 numpy (exact)."""
    return t.view(torch.bfloat16).to(torch.float64).cpu().numpy()


def bf16_bits_of(ref):
    """float64 numpy -> bf16 bits (round to nearest even) via torch's cast of exact float32 values."""
    return torch.from_numpy(np.asarray(ref, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
