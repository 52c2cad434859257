"""Calls from several host threads at once, each thread on its own stream.
The library serialises its entry points with one lock, hands dependency
words to every thread's calls from one sequence, and keeps the last error
per thread. Every output must equal a single-threaded reference bit for
bit, and a failing call on one thread must leave the others' error state
alone."""
import threading

import pytest
import torch

import comm_overlapped_linear_amd as tp
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty

pytestmark = pytest.mark.gpu

CALLS = 30
# staged over several internal streams (explicit grouping), the remote run
# passing the last slice (rank 1 of 4)
AG = W.AgCase("threads_ag_bf16_p4", M=4 * 256, N=512, K=512, P=4, rank=1, dist="u11")
RS = W.RsCase("threads_rs_bf16_p4", M=4 * 256, N=512, K=256, P=4, rank=2, std=0.5)


def test_calls_from_several_threads():
    ag_in = W.ag_inputs(AG)
    slices = [dev(s) for s in ag_in["a_slices"]]
    b, c = dev(ag_in["b"]), dev(ag_in["c"])
    rs_in = W.rs_inputs(RS)
    ra, rb = dev(rs_in["a"]), dev(rs_in["b"])
    inc = [dev(x) if x is not None else None for x in rs_in["incoming"]]
    ag_kw = dict(M=AG.M, N=AG.N, K=AG.K, rank=AG.rank, alpha=AG.alpha, beta=AG.beta, groups=1)
    rs_kw = dict(M=RS.M, N=RS.N, K=RS.K, P=RS.P, rank=RS.rank, groups=1)

    say("threads: single-threaded references")
    ag_ref, rs_ref = bf16_empty(AG.M, AG.N), bf16_empty(RS.M, RS.N)
    tp.stage_ag(slices, b, c, ag_ref, **ag_kw)
    tp.stage_rs(ra, rb, inc, rs_ref, **rs_kw)
    torch.cuda.synchronize()
    ag_ref, rs_ref = ag_ref.cpu(), rs_ref.cpu()

    outs, errors, last = {}, {}, {}

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            if i % 2 == 0:
                d = bf16_empty(AG.M, AG.N)
                call = tp.prepare_stage_ag(slices, b, c, d, **ag_kw)
            else:
                d = bf16_empty(RS.M, RS.N)
                call = tp.prepare_stage_rs(ra, rb, inc, d, **rs_kw)
            bad = torch.zeros(1, dtype=torch.int64, device="cuda")
            first = None
            for n in range(CALLS):
                call(stream=stream)
                with torch.cuda.stream(stream):
                    if first is None:
                        first = d.clone()
                    bad.add_((d != first).sum())
                if i == 3 and n == CALLS // 2:
                    # a failing call on this thread only (rank out of range)
                    with pytest.raises(tp.TpgError):
                        tp.stage_ag(slices, b, c, bf16_empty(AG.M, AG.N), **dict(ag_kw, rank=AG.P))
            stream.synchronize()
            outs[i] = (first.cpu(), int(bad.item()))
            last[i] = tp.last_error()
        except BaseException as e:      # reported by the main thread
            errors[i] = e

    say(f"threads: 4 threads x {CALLS} calls")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, (first, bad) in outs.items():
        ref = ag_ref if i % 2 == 0 else rs_ref
        assert torch.equal(first, ref), f"thread {i}: differs from the single-threaded call"
        assert bad == 0, f"thread {i}: {bad} elements changed between calls"
    # the failing call's message stays on its own thread (3); a later good
    # call there clears it, so every thread ends with an empty error
    assert all(msg == "" for msg in last.values()), last
