"""The allocation-free all-gather entry point (tpgemm_stage_ag_noalloc)
through the C ABI: on calls in a row, the second with a smaller input (the
static scratch then still holds the first call's slices), its output equals
tpgemm_stage_ag's bit for bit and matches the oracle; sizes past the static
scratch and graph / profile flags are rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

# first a larger call (7 MiB of receive slots, two full-chip launches), then
# smaller ones: two with in-kernel gates (a copy kernel beside the GEMM, then
# a latency-bound call carrying its copy), a bf16 call on the register-staged
# kernel (K * 2 bytes not a multiple of 128), a latency-bound one on one
# stream, and an unstaged one
SEQUENCE = [
    (W.AgCase("noalloc_e4m3_p8", M=8 * 512, N=1024, K=2048, P=8, rank=3, dtype="e4m3", dist="n05",
              c_dist="n01"), 0),
    # in-kernel gates: counters in the static scratch after the slots, both forms
    (W.AgCase("noalloc_e4m3_p4_in_kernel_gates", M=4 * 256, N=512, K=2048, P=4, rank=2, dtype="e4m3",
              dist="n05", c_dist="n01"), tp.IN_KERNEL_GATES),
    (W.AgCase("noalloc_bf16_p4_in_kernel_gates_carried", M=4 * 128, N=256, K=256, P=4, rank=1, dist="u11"),
     tp.IN_KERNEL_GATES),
    (W.AgCase("noalloc_bf16_p4_small", M=4 * 136, N=264, K=200, P=4, rank=1, dist="u11", alpha=0.5,
              beta=-1.0), 0),
    (W.AgCase("noalloc_bf16_p2_latency", M=2 * 128, N=256, K=512, P=2, rank=1, dist="u11"), 0),
    (W.AgCase("noalloc_bf16_p4_unstaged", M=4 * 72, N=200, K=256, P=4, rank=2, dist="n05", beta=0.0), tp.UNSTAGED),
]


def _kw(case):
    return dict(M=case.M, N=case.N, K=case.K, rank=case.rank, dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
                alpha=case.alpha, beta=case.beta)


def test_noalloc_matches_stage_ag_on_calls_in_a_row():
    for case, flags in SEQUENCE:
        say(f"noalloc: {case.name} flags={flags}")
        inp = W.ag_inputs(case)
        ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank, case.dtype)
        slices = [dev(s) for s in inp["a_slices"]]
        b, c = dev(inp["b"]), dev(inp["c"])
        d_ref = bf16_empty(case.M, case.N)
        tp.stage_ag(slices, b, c, d_ref, flags=flags, **_kw(case))
        d = bf16_empty(case.M, case.N)
        tp.stage_ag_noalloc(slices, b, c, d, flags=flags, **_kw(case))
        torch.cuda.synchronize()
        assert torch.equal(d.cpu(), d_ref.cpu()), case.name
        assert_parity(host_f64(d), ref, case.name)


def test_noalloc_rejects_before_enqueue():
    case = W.AgCase("noalloc_too_big", M=8 * 1280, N=256, K=8192, P=8, dtype="e4m3", dist="n05", beta=0.0)
    m = case.m
    slices = [torch.zeros((m, case.K), dtype=torch.uint8, device="cuda") for _ in range(case.P)]
    b = torch.zeros((case.N, case.K), dtype=torch.uint8, device="cuda")
    d = bf16_empty(case.M, case.N)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, None, d, **_kw(case)))
    assert need > 64 << 20
    with pytest.raises(tp.TpgError) as e:
        tp.stage_ag_noalloc(slices, b, None, d, **_kw(case))
    assert e.value.status == tp.ERR_WORKSPACE
    small = W.AgCase("noalloc_flags", M=2 * 64, N=128, K=128, P=2, dist="u11", beta=0.0)
    sl = [torch.zeros((64, 128), dtype=torch.int16, device="cuda") for _ in range(2)]
    bb = torch.zeros((128, 128), dtype=torch.int16, device="cuda")
    dd = bf16_empty(128, 128)
    for flags in (tp.FORCE_GRAPH, tp.PROFILE):
        with pytest.raises(tp.TpgError) as e:
            tp.stage_ag_noalloc(sl, bb, None, dd, flags=flags, **_kw(small))
        assert e.value.status == tp.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.isnan(host_f64(dd)).all()     # nothing was enqueued
