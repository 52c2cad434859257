"""GPU parity past the 32-bit limits: operands and outputs larger than 2^31
bytes or elements, through the C ABI.

* Weights of more than 2 GiB: the direct-to-LDS kernel addresses B with
  31-bit offsets, so this call takes the register-staged kernel with 64-bit
  addressing. Small-integer operands make every fp32 sum exact, so sampled
  output columns (including those whose weight rows start past 2 GiB) must
  equal the oracle's value rounded once to bf16, bit for bit.
* An output of more than 2^31 elements (4.3 GB) on the direct-to-LDS kernel,
  with a ragged last tile row and column: sampled rows (the last ones past
  element 2^31) against the oracle, no element left unwritten, and the staged
  call equal to the unstaged one bit for bit.
"""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import gen
from tests.devutil import say, dev, bf16_empty, host_f64, bf16_bits_of
from tests.parity import assert_parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_ag_weights_beyond_2gib_are_exact():
    P, rank, m, N, K = 2, 1, 128, 32776, 65536
    M = P * m
    assert N * K > 2 ** 31
    say("large: weights beyond 2 GiB generate")
    key = lambda tag, s=0: gen.stream_key(4100 + s, tag)
    a_slices = [gen.encode_e4m3(gen.small_ints(key("a", s), m * K, -2, 2).astype(np.float64)).reshape(m, K)
                for s in range(P)]
    b = gen.shifted_rows(key("b"), N, K, -2, 2, gen.encode_e4m3, np.uint8)
    da = [dev(s) for s in a_slices]
    db = dev(b)
    kw = dict(M=M, N=N, K=K, rank=rank, dtype=tp.E4M3, alpha=1.0, beta=0.0)
    d = bf16_empty(M, N)
    say("large: weights beyond 2 GiB staged")
    tp.stage_ag(da, db, None, d, **kw)
    torch.cuda.synchronize()
    assert not torch.isnan(d.view(torch.bfloat16)).any().item()
    cols = sorted({0, 1, 255, 256, 16383, 16384, 32766, 32767, 32768, 32769, *range(N - 8, N),
                   *np.random.default_rng(3).integers(0, N, 32).tolist()})
    say("large: weights beyond 2 GiB oracle")
    ref = oracle.gemm_ag(a_slices, b[cols], None, 1.0, 0.0, rank, dtype="e4m3", b_layout="nk")
    got = d[:, torch.tensor(cols, device="cuda")].cpu().numpy()
    assert np.array_equal(got, bf16_bits_of(ref))
    d2 = bf16_empty(M, N)
    say("large: weights beyond 2 GiB unstaged")
    tp.stage_ag(da, db, None, d2, flags=tp.UNSTAGED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(d, d2)


def test_ag_output_beyond_2g_elements():
    P, rank, m, N, K = 2, 0, 32832, 32776, 128
    M = P * m
    assert M * N > 2 ** 31
    say("large: output beyond 2^31 elements generate")
    key = lambda tag, s=0: gen.stream_key(4200 + s, tag)
    a_slices = [gen.normal_bf16(key("a", s), (m, K)) for s in range(P)]
    b = gen.normal_bf16(key("b"), (N, K), 0.0, 0.1)
    da = [dev(s) for s in a_slices]
    db = dev(b)
    kw = dict(M=M, N=N, K=K, rank=rank, alpha=0.5, beta=0.0)
    d = bf16_empty(M, N)
    say("large: output beyond 2^31 elements staged")
    tp.stage_ag(da, db, None, d, **kw)
    torch.cuda.synchronize()
    assert not torch.isnan(d.view(torch.bfloat16)).any().item()
    rows = sorted({0, m - 1, m, M - 65, *range(M - 64, M),
                   *np.random.default_rng(4).integers(0, M, 40).tolist()})
    assert rows[-1] * N >= 2 ** 31
    say("large: output beyond 2^31 elements oracle")
    ref = oracle.gemm_ag_rows(a_slices, b, None, 0.5, 0.0, "bf16", "nk", rows)
    assert_parity(host_f64(d[torch.tensor(rows, device="cuda")]), ref, "output beyond 2^31 elements")
    d2 = bf16_empty(M, N)
    say("large: output beyond 2^31 elements unstaged")
    tp.stage_ag(da, db, None, d2, flags=tp.UNSTAGED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(d, d2)
