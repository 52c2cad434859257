"""GPU parity of launches whose tile order the launcher fixes: one round of
tiles split evenly over the 8 XCDs, where each XCD's run of tiles is made one
whole rectangle (group heights 1, 4, 6 and 7 tile-rows here, with ragged last
tile rows and columns). Small-integer operands make every fp32 sum exact, so
each element must equal the oracle's value rounded once to bf16, bit for bit:
a tile that is skipped, or placed at the wrong rows or columns, cannot pass."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import gen
from tests.devutil import say, dev, bf16_empty, bf16_bits_of

pytestmark = pytest.mark.gpu

# (M, N, K, P, dtype): 128 x 256 tiles give 28 x 4, 28 x 4 (ragged), 56 x 4,
# 16 x 4 and 12 x 8 tile grids
SHAPES = [(3584, 1024, 256, 1, "bf16"), (3544, 1000, 256, 2, "bf16"), (7168, 1024, 128, 1, "e4m3"),
          (2048, 1024, 256, 2, "e4m3"), (1536, 2048, 128, 1, "bf16")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:3])) + f"_p{s[3]}_{s[4]}")
def test_one_round_tile_orders_are_exact(shape):
    M, N, K, P, dtype = shape
    m = M // P
    assert m * P == M
    enc = gen.encode_e4m3 if dtype == "e4m3" else gen.encode_bf16
    key = lambda tag, s=0: gen.stream_key(4300 + M + N + s, tag)
    a_slices = [enc(gen.small_ints(key("a", s), m * K, -2, 2).astype(np.float64)).reshape(m, K) for s in range(P)]
    b = enc(gen.small_ints(key("b"), N * K, -2, 2).astype(np.float64)).reshape(N, K)
    c = gen.encode_bf16(gen.small_ints(key("c"), M * N, -3, 3).astype(np.float64)).reshape(M, N)
    ref_bits = bf16_bits_of(oracle.gemm_ag(a_slices, b, c, 1.0, 1.0, P - 1, dtype=dtype, b_layout="nk"))
    for flags in (0, tp.UNSTAGED):
        say(f"tile order: {shape} flags={flags}")
        d = bf16_empty(M, N)
        tp.stage_ag([dev(s) for s in a_slices], dev(b), dev(c), d, M=M, N=N, K=K, rank=P - 1,
                    dtype=tp.E4M3 if dtype == "e4m3" else tp.BF16, alpha=1.0, beta=1.0, flags=flags)
        torch.cuda.synchronize()
        assert np.array_equal(d.cpu().numpy(), ref_bits), (shape, flags)
