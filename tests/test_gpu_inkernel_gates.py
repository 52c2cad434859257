"""The staged all-gather as one launch (TPG_IN_KERNEL_GATES): parity with the
oracle and bitwise identity with the event-gated schedule, with deliveries
held back 20 ms behind a host callback while the GEMM's tiles are already
waiting on their chunk counters, receive slots poisoned with NaN, and the
counters left full by a previous call (the call must zero them first).
The negative control drops the in-kernel waits and must then read NaN."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

HOLD = tp.DEBUG_HOLD_DELIVERIES
IKG = tp.IN_KERNEL_GATES

# M/P a multiple of 128 and K * element bytes a multiple of 128. K-steps of
# 128 bytes, in at most 8 chunks: 4 chunks of 1 step (bf16 K=256), 5 of 1
# (K=320), 5 chunks of 2 with a ragged last one (e4m3 K=1152), 8 of 4 (bf16
# K=2048); the last case has several tiles per persistent workgroup. The
# other cases are latency-bound: without the host hold their deliveries ride
# in the GEMM launch itself (one counter for all of them).
CASES = [
    W.AgCase("ikg_bf16_p8", M=8 * 128, N=264, K=256, P=8, rank=3, dist="u11"),
    W.AgCase("ikg_bf16_p4_kn", M=4 * 128, N=272, K=320, P=4, rank=1, b_layout="kn", alpha=0.5, beta=-1.0),
    W.AgCase("ikg_e4m3_p4_ragged_chunk", M=4 * 256, N=200, K=1152, P=4, rank=2, dtype="e4m3", dist="n05",
             c_dist="n01"),
    W.AgCase("ikg_bf16_p2_swiglu", M=2 * 128, N=2 * 136, K=2048, P=2, rank=1, swiglu=True, beta=0.0),
    W.AgCase("ikg_bf16_p8_many_tiles_per_wg", M=8 * 512, N=4096, K=256, P=8, rank=6, dist="u11", beta=0.0),
]


def poisoned(nbytes, elem_bytes):
    """A workspace whose every element is a NaN of the operand type."""
    if elem_bytes == 2:
        return torch.full((max(nbytes, 2) // 2,), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint8)
    return torch.full((max(nbytes, 1),), 0x7F, dtype=torch.uint8, device="cuda")   # e4m3 NaN


def call(case, slices, b, c, flags, ws=None, rank=None):
    nout = case.N // 2 if case.swiglu else case.N
    d = bf16_empty(case.M, nout)
    tp.stage_ag(slices, b, c, d, M=case.M, N=case.N, K=case.K, rank=case.rank if rank is None else rank,
                dtype=tp.E4M3 if case.dtype == "e4m3" else tp.BF16,
                b_layout=tp.B_KN if case.b_layout == "kn" else tp.B_NK,
                epilogue=tp.EPI_SWIGLU if case.swiglu else tp.EPI_ALPHA_BETA,
                alpha=case.alpha, beta=case.beta, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    return d


def setup(case):
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank,
                         case.dtype, case.b_layout, swiglu=case.swiglu)
    slices = [dev(s) for s in inp["a_slices"]]
    b = dev(inp["b"])
    c = dev(inp["c"]) if inp["c"] is not None else None
    return ref, slices, b, c


def slot_bytes(case):
    eb = 1 if case.dtype == "e4m3" else 2
    return (case.P - 1) * case.m * case.K * eb


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_in_kernel_gates_parity_and_identity(case):
    ref, slices, b, c = setup(case)
    eb = 1 if case.dtype == "e4m3" else 2
    say(f"in-kernel gates: {case.name} event-gated reference")
    base = call(case, slices, b, c, tp.NO_GRAPH)
    nout = case.N // 2 if case.swiglu else case.N
    probe = bf16_empty(case.M, nout)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, probe, M=case.M, N=case.N, K=case.K,
                                                 rank=case.rank, flags=IKG,
                                                 dtype=tp.E4M3 if eb == 1 else tp.BF16))
    assert need >= slot_bytes(case) + 256
    ws = poisoned(need, eb)
    # in place (TPG_NO_COPY) the slices must be back to back
    whole = torch.cat(slices)
    views = [whole[i * case.m:(i + 1) * case.m] for i in range(case.P)]
    for flags in (IKG, IKG | HOLD, IKG | HOLD | tp.FORCE_GRAPH, IKG | tp.NO_COPY):
        say(f"in-kernel gates: {case.name} flags={flags}")
        # slots poisoned again, counters as the previous call left them
        ws[:slot_bytes(case)] = poisoned(slot_bytes(case), eb)
        d = call(case, views if flags & tp.NO_COPY else slices, b, c, flags, ws)
        got = host_f64(d)
        assert not np.isnan(got).any(), f"{case.name}/flags={flags}: a tile read an undelivered chunk"
        assert_parity(got, ref, f"{case.name}/flags={flags}")
        assert torch.equal(d.cpu(), base.cpu()), f"{case.name}/flags={flags}: differs from the event-gated run"


def test_in_kernel_gates_every_rank():
    case = CASES[0]
    inp = W.ag_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    for r in range(case.P):
        ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, r)
        # deliveries carried by the GEMM launch (a latency-bound call), and on
        # a stream of their own behind the host hold
        for flags in (IKG, IKG | HOLD):
            say(f"in-kernel gates: rank {r} flags={flags}")
            d = call(case, slices, b, c, flags, rank=r)
            assert_parity(host_f64(d), ref, f"rank {r}/flags={flags}")


def test_in_kernel_gates_negative_control():
    """Without the in-kernel waits the remote slices' tiles read the poisoned
    slots long before the held deliveries land: their rows must be NaN, the
    local slice's rows right."""
    case = CASES[0]
    ref, slices, b, c = setup(case)
    probe = bf16_empty(case.M, case.N)
    need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, probe, M=case.M, N=case.N, K=case.K,
                                                 rank=case.rank, flags=IKG))
    ws = poisoned(need, 2)
    say("in-kernel gates: negative control")
    d = call(case, slices, b, c, IKG | HOLD | tp.DEBUG_NO_GATE, ws)
    got = host_f64(d)
    m = case.m
    for s in range(case.P):
        rows = slice(s * m, (s + 1) * m)
        if s == case.rank:
            assert_parity(got[rows], ref[rows], "local slice")
        else:
            assert np.isnan(got[rows]).all(), f"slice {s} read its slot after the delivery"


def test_in_kernel_gates_bounded_wait():
    """The bounded wait, forced from the host: every in-kernel wait asks for
    one arrival more than will come and gives up after 20 us. Every tile of
    a delivered slice must then write NaN (never a silent wrong value), the
    local slice's rows stay right, and the call ends at once: the kernels
    exit. Both forms: deliveries carried in the GEMM launch, and on their own
    stream behind the host hold."""
    import time
    case = CASES[0]
    ref, slices, b, c = setup(case)
    m = case.m
    for flags in (IKG | tp.DEBUG_GATE_TIMEOUT, IKG | tp.DEBUG_GATE_TIMEOUT | HOLD):
        say(f"in-kernel gates: bounded wait flags={flags}")
        t0 = time.perf_counter()
        d = call(case, slices, b, c, flags)
        assert time.perf_counter() - t0 < 5.0
        got = host_f64(d)
        for s in range(case.P):
            rows = slice(s * m, (s + 1) * m)
            if s == case.rank:
                assert_parity(got[rows], ref[rows], "local slice")
            else:
                assert np.isnan(got[rows]).all(), f"slice {s}: a tile that gave up did not write NaN"


def test_static_words_survive_release_caches():
    """The library's static gate and dependency words keep their last values
    when tpg_release_caches drops the per-device contexts, so the host's
    record of them (the numbers that stamp the dependency words, the totals
    the gate counters have reached) must survive too: a wait would otherwise
    pass at once or never. With the deliveries held 20 ms behind the host and
    the receive slots poisoned, a run that passed its wait early reads NaN.
    Both forms: the staged schedule on several streams (stream memory
    operations between them) and the latency-bound call carrying its
    deliveries (one gate counter)."""
    staged = CASES[4]
    for case, flags in ((staged, HOLD), (CASES[0], 0)):
        ref, slices, b, c = setup(case)
        probe = bf16_empty(case.M, case.N)
        need = tp.stage_ag_workspace_size(tp.ag_args(slices, b, c, probe, M=case.M, N=case.N, K=case.K,
                                                     rank=case.rank, flags=flags))
        ws = poisoned(need, 2)
        outs = []
        for life in range(2):
            say(f"static words: {case.name} flags={flags} life {life}")
            ws[:slot_bytes(case)] = poisoned(slot_bytes(case), 2)
            d = call(case, slices, b, c, flags | tp.NO_GRAPH, ws)
            got = host_f64(d)
            assert not np.isnan(got).any(), f"{case.name}/life {life}: a wait passed before its delivery"
            assert_parity(got, ref, f"{case.name}/life {life}")
            outs.append(d.cpu())
            tp.release_caches()
        assert torch.equal(outs[0], outs[1])
