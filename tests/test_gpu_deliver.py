"""The stage delivery as its own call (tpg_deliver): every copy kind moves
the bytes exactly, with strided receive slots, slices of any size (the
library's kernel takes 16-byte multiples, other sizes go to the runtime's
copy) and slices adjacent in memory."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
from tests.devutil import say

pytestmark = pytest.mark.gpu

KINDS = {"default": 0, "kernel": tp.COPY_KERNEL, "shader": tp.COPY_SHADER, "sdma": tp.COPY_SDMA}


@pytest.mark.parametrize("nbytes,n,pad", [(8 << 20, 7, 0), (1 << 20, 3, 256), (4096 + 16, 5, 0), (1000, 4, 24),
                                          (16, 1, 0), (3 << 20, 64, 0)])
@pytest.mark.parametrize("kind", list(KINDS))
def test_deliver_is_exact(nbytes, n, pad, kind):
    rng = np.random.default_rng(nbytes + n)
    srcs = [torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda() for _ in range(n)]
    stride = nbytes + pad
    dst = torch.full((stride * n,), 0xA5, dtype=torch.uint8, device="cuda")
    say(f"deliver: {kind} n={n} bytes={nbytes} stride={stride}")
    tp.deliver(srcs, dst, nbytes=nbytes, dst_stride=stride, flags=KINDS[kind])
    torch.cuda.synchronize()
    got = dst.view(n, stride)
    for i in range(n):
        assert torch.equal(got[i, :nbytes], srcs[i]), i
        assert bool((got[i, nbytes:] == 0xA5).all())      # the padding is untouched


def test_deliver_adjacent_slices():
    """Slices that sit back to back in one buffer (merged into one runtime
    copy by the shader and copy-engine kinds)."""
    big = torch.arange(6 * 4096, dtype=torch.int32, device="cuda").view(torch.uint8)
    nb = 4 * 4096
    srcs = [big[i * nb:(i + 1) * nb] for i in range(6)]
    for kind, fl in KINDS.items():
        dst = torch.zeros(6 * nb, dtype=torch.uint8, device="cuda")
        tp.deliver(srcs, dst, nbytes=nb, flags=fl)
        torch.cuda.synchronize()
        assert torch.equal(dst, big), kind
