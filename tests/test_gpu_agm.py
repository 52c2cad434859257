"""GPU parity of several projections sharing one all-gathered input
(tpgemm_stage_ag_multi, the fused QKV form) against the oracle, through the C
ABI: every issue mode and stage grouping, weights apart (copied side by
side) and back to back (read in place), an empty projection, and bitwise
equality with the single-weight call on the concatenated weights."""
import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

MODES = {"default": 0, "graph": tp.FORCE_GRAPH, "eager": tp.NO_GRAPH, "unstaged": tp.UNSTAGED,
         "no_copy": tp.NO_COPY, "serial": tp.SERIAL_STAGES, "sdma": tp.COPY_SDMA, "shader": tp.COPY_SHADER}


def dt_of(case):
    return tp.E4M3 if case.dtype == "e4m3" else tp.BF16


def run(case, slices, bs, flags=0, groups=0, ns=None):
    ds = [bf16_empty(case.M, n) for n in case.ns]
    tp.stage_ag_multi(slices, bs, ds, M=case.M, K=case.K, ns=ns, rank=case.rank, dtype=dt_of(case),
                      alpha=case.alpha, flags=flags, groups=groups)
    torch.cuda.synchronize()
    return ds


@pytest.mark.parametrize("case", W.SMALL_AGM, ids=lambda c: c.name)
def test_ag_multi_parity_all_modes(case):
    inp = W.ag_multi_inputs(case)
    refs = oracle.gemm_ag_multi(inp["a_slices"], inp["bs"], case.alpha, case.rank, case.dtype)
    slices = [dev(s) for s in inp["a_slices"]]
    apart = [dev(b) for b in inp["bs"]]
    whole = dev(np.concatenate(inp["bs"], axis=0))
    offs = np.cumsum([0] + list(case.ns))
    adjacent = [whole[offs[i]:offs[i + 1]] for i in range(len(case.ns))]
    first = None
    for wname, bs in (("apart", apart), ("adjacent", adjacent)):
        for name, flags in MODES.items():
            for groups in sorted({0, 1, 2, case.P - 1}):
                if name == "no_copy" and groups == 0 and flags & tp.UNSTAGED:
                    continue
                say(f"ag multi: {case.name} weights={wname} mode={name} groups={groups}")
                ds = run(case, slices, bs, flags, groups)
                for i, (d, ref) in enumerate(zip(ds, refs)):
                    assert_parity(host_f64(d), ref, f"{case.name}/{wname}/{name}/{groups}/out{i}")
                if first is None:
                    first = [d.cpu() for d in ds]
                for d, f in zip(ds, first):          # row partitions of one product: the same bits
                    assert torch.equal(d.cpu(), f), (wname, name, groups)
    # the single-weight call on the concatenated weights gives the same bits
    d = bf16_empty(case.M, sum(case.ns))
    tp.stage_ag(slices, whole, None, d, M=case.M, N=sum(case.ns), K=case.K, rank=case.rank, dtype=dt_of(case),
                alpha=case.alpha, beta=0.0)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(first, dim=1), d.cpu())


def test_ag_multi_empty_projection_is_untouched():
    case = W.AgmCase("agm_empty", M=4 * 64, K=256, P=4, ns=(64, 0, 24), rank=2)
    inp = W.ag_multi_inputs(W.AgmCase("x", M=case.M, K=case.K, P=4, ns=(64, 8, 24), rank=2))
    bs = [dev(inp["bs"][0]), dev(inp["bs"][1]), dev(inp["bs"][2])]
    ds = [bf16_empty(case.M, 64), bf16_empty(case.M, 8), bf16_empty(case.M, 24)]
    say("ag multi: empty middle projection")
    tp.stage_ag_multi([dev(s) for s in inp["a_slices"]], bs, ds, M=case.M, K=case.K, ns=(64, 0, 24), rank=2)
    torch.cuda.synchronize()
    refs = oracle.gemm_ag_multi(inp["a_slices"], [inp["bs"][0], inp["bs"][2]], 1.0, 2)
    assert_parity(host_f64(ds[0]), refs[0], "out0")
    assert_parity(host_f64(ds[2]), refs[1], "out2")
    assert bool((ds[1] == 0x7FC0).all())                    # still the NaN fill


def test_ag_multi_graph_replay_sees_new_data():
    case = W.SMALL_AGM[0]
    inp = W.ag_multi_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    bs = [dev(b) for b in inp["bs"]]
    ds = [bf16_empty(case.M, n) for n in case.ns]
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for it in range(3):
        say(f"ag multi: graph replay {it}")
        tp.stage_ag_multi(slices, bs, ds, M=case.M, K=case.K, rank=case.rank, flags=tp.FORCE_GRAPH, workspace=ws)
        torch.cuda.synchronize()
        refs = oracle.gemm_ag_multi([s.cpu().numpy().view(np.uint16) for s in slices],
                                    [b.cpu().numpy().view(np.uint16) for b in bs], 1.0, case.rank)
        for d, ref in zip(ds, refs):
            assert_parity(host_f64(d), ref, f"replay {it}")
        for s in slices:
            s.copy_(torch.roll(s, 1, dims=0))
