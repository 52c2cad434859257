"""The library's static word arrays under reuse: the token-stamped gate words
(65536, one per latency-bound call that carries its deliveries) and the
dependency words (65536, one per cross-stream dependency of an eager call).
More calls than words are issued on two streams while one of them starts
behind a 200 ms spin kernel, so the host runs ahead of the device and calls
queue up on both streams. Every call's output must be right, and the run
must end."""
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

GATE_WORDS = 65536
SYNC_WORDS = 65536
HOLD_CYCLES = 400_000_000          # about 200 ms of the shader clock


def prepared_pair(case, inp, groups=0):
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    outs, calls = [], []
    for _ in range(2):             # one output and workspace per stream
        d = bf16_empty(case.M, case.N)
        calls.append(tp.prepare_stage_ag(slices, b, c, d, M=case.M, N=case.N, K=case.K, rank=case.rank,
                                         alpha=case.alpha, beta=case.beta, groups=groups))
        outs.append(d)
    return calls, outs, (slices, b, c)


def test_gate_words_reused_across_streams():
    """Latency-bound calls carrying their deliveries, each output compared
    with the first on the device."""
    case = W.C1
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank)
    calls, outs, keep = prepared_pair(case, inp)
    calls[0]()
    torch.cuda.synchronize()
    assert_parity(host_f64(outs[0]), ref, case.name)
    first = outs[0].clone()
    bad = torch.zeros(2, dtype=torch.int64, device="cuda")    # one count per stream
    n = GATE_WORDS + 200
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say(f"words: {n} carried calls over two streams, one held")
    with torch.cuda.stream(streams[0]):
        torch.cuda._sleep(HOLD_CYCLES)
    for i in range(n):
        k = i % 2
        calls[k](stream=streams[k])
        with torch.cuda.stream(streams[k]):
            bad[k].add_((outs[k] != first).sum())
        if i % 16000 == 0:
            say(f"words: call {i}")
    torch.cuda.synchronize()
    assert bad.sum().item() == 0


def test_dependency_words_reused_across_streams():
    """Staged calls on several streams (fork and join as stream memory
    operations), each output compared with the first on the device."""
    case = W.AgCase("words_bf16_p2", M=2 * 512, N=1024, K=512, P=2, rank=1, dist="u11")
    assert 2.0 * case.M * case.N * case.K >= 1e9       # not latency-bound: a staged call on two streams
    inp = W.ag_inputs(case)
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank)
    calls, outs, keep = prepared_pair(case, inp, groups=1)   # one explicit run: never the one-launch form
    calls[0]()
    torch.cuda.synchronize()
    assert_parity(host_f64(outs[0]), ref, case.name)
    first = outs[0].clone()
    bad = torch.zeros(2, dtype=torch.int64, device="cuda")    # one count per stream
    n = SYNC_WORDS + 500            # at least one dependency per call (the join)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say(f"words: {n} staged calls over two streams, one held")
    with torch.cuda.stream(streams[0]):
        torch.cuda._sleep(HOLD_CYCLES)
    for i in range(n):
        k = i % 2
        calls[k](stream=streams[k])
        with torch.cuda.stream(streams[k]):
            bad[k].add_((outs[k] != first).sum())
        if i % 16000 == 0:
            say(f"words: call {i}")
    torch.cuda.synchronize()
    assert bad.sum().item() == 0
