"""Full-size GPU parity: the five workloads at their real shapes, in the launch
configuration the benchmark times (the library's default issue and copy kind
for each call).

The float64 oracle computes every output element (BLAS products on the
host's cores: about 1 s for the e4m3 all-gather, 4 s for the reduce-scatter,
20 s for the FFN layer), and every element is held to the tolerance. On top,
properties that hold at any size: staged equals unstaged bit for bit, and
the own reduce-scatter block minus the incoming partials equals the plain
partial at a tolerance scaled to that partial.
"""
import dataclasses

import numpy as np
import pytest
import torch

import comm_overlapped_linear_amd as tp
import oracle
from synth import workloads as W
from tests.devutil import say, dev, bf16_empty, host_f64
from tests.parity import assert_parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


# rank 3 of 8: the remote run passes slice 7 and goes on from slice 0, one
# launch whose tiles past the wrap write 8192 rows earlier
@pytest.mark.parametrize("case", [W.C2, W.C2_BETA0, dataclasses.replace(W.C2, name=W.C2.name + "_rank3", rank=3)],
                         ids=lambda c: c.name)
def test_full_ag_fp8(case):
    say(f"full: {case.name} generate")
    inp = W.ag_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    b, c = dev(inp["b"]), dev(inp["c"])
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, dtype=tp.E4M3, alpha=case.alpha, beta=case.beta)
    d = bf16_empty(case.M, case.N)
    say(f"full: {case.name} staged")
    tp.stage_ag(slices, b, c, d, **kw)
    torch.cuda.synchronize()
    say(f"full: {case.name} oracle")
    ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, case.rank, "e4m3", "nk")
    assert_parity(host_f64(d), ref, case.name)
    d2 = bf16_empty(case.M, case.N)
    say(f"full: {case.name} unstaged")
    tp.stage_ag(slices, b, c, d2, flags=tp.UNSTAGED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(d, d2)


# rank 4 of 8: the emitted blocks 5, 6, 7, 0, 1, 2, 3 as one launch whose
# tiles past block 7 read A and write D 8192 rows earlier
@pytest.mark.parametrize("case", [W.C3, dataclasses.replace(W.C3, name=W.C3.name + "_rank4", rank=4)],
                         ids=lambda c: c.name)
def test_full_rs_bf16(case):
    say(f"full: {case.name} generate")
    inp = W.rs_inputs(case)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    kw = dict(M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank)
    d = bf16_empty(case.M, case.N)
    say(f"full: {case.name} staged")
    tp.stage_rs(a, b, inc, d, **kw)
    torch.cuda.synchronize()
    got = host_f64(d)
    say(f"full: {case.name} oracle")
    ref = oracle.gemm_rs(inp["a"], inp["b"], inp["incoming"], 1.0, case.rank, case.P)
    for blk in range(case.P):           # tolerance per block
        rows = slice(blk * case.m, (blk + 1) * case.m)
        assert_parity(got[rows], ref[rows], f"block {blk}")
    # own partial inside the reduced block, at a tolerance scaled to the partial itself
    own = slice(case.rank * case.m, (case.rank + 1) * case.m)
    inc_sum = sum(oracle.decode_bf16(x) for x in inp["incoming"] if x is not None)
    e_r = oracle.gemm_rs_rows(inp["a"], inp["b"], None, 1.0, case.rank, case.P, "nk",
                              list(range(own.start, own.stop)))
    ulp_out = np.exp2(np.floor(np.log2(np.maximum(np.abs(got[own]), 1e-30))) - 7)
    assert np.all(np.abs(got[own] - inc_sum - e_r) <= 0.02 * np.sqrt(np.mean(e_r ** 2)) + ulp_out)
    d2 = bf16_empty(case.M, case.N)
    say(f"full: {case.name} unstaged")
    tp.stage_rs(a, b, inc, d2, flags=tp.UNSTAGED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(d, d2)


def test_full_ffn():
    case = W.C4
    say(f"full: {case.name} generate")
    inp = W.ffn_inputs(case)
    t = {k: dev(v) for k, v in inp.items()}
    y = bf16_empty(case.PB, case.L, case.D)
    say(f"full: {case.name} run")
    tp.ffn_slot_forward(t["x"], t["w1"], t["b1"], t["wout"], t["bout"], t["gx"], t["bx"], t["gg"], t["bg"], y,
                        PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps)
    torch.cuda.synchronize()
    got = host_f64(y)
    say(f"full: {case.name} oracle")
    ref = oracle.ffn_slot_forward(inp, case.eps)
    assert_parity(got, ref, case.name)
    y2 = bf16_empty(case.PB, case.L, case.D)
    tp.ffn_slot_forward(t["x"], t["w1"], t["b1"], t["wout"], t["bout"], t["gx"], t["bx"], t["gg"], t["bg"], y2,
                        PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps, flags=tp.SERIAL_STAGES)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_full_swiglu_block():
    case = W.C5
    say(f"full: {case.name} generate")
    inp = W.swiglu_inputs(case)
    xs = [dev(x) for x in inp["x_shards"]]
    w13, w2 = dev(inp["w13"]), dev(inp["w2"])
    h = bf16_empty(case.M, case.F)
    out = bf16_empty(case.M, case.D)
    say(f"full: {case.name} run")
    tp.stage_ag(xs, w13, None, h, M=case.M, N=2 * case.F, K=case.D, rank=case.rank, b_layout=tp.B_KN,
                epilogue=tp.EPI_SWIGLU, alpha=1.0, beta=0.0)
    tp.stage_rs(h, w2, None, out, M=case.M, N=case.D, K=case.F, P=case.P, rank=case.rank, b_layout=tp.B_KN)
    torch.cuda.synchronize()
    say(f"full: {case.name} oracle")
    h_ref = oracle.swiglu_hidden(inp["x_shards"], inp["w13"])
    assert_parity(host_f64(h), h_ref, "h")
    out_ref = h_ref @ oracle.decode_bf16(inp["w2"])
    for blk in range(case.P):           # the reduce-scatter blocks
        rows = slice(blk * case.S, (blk + 1) * case.S)
        assert_parity(host_f64(out)[rows], out_ref[rows], f"partial block {blk}")


def test_full_ag_rotb_e4m3():
    """Rotating B at the e4m3 all-gather shape: A local (8192 x 8192), B as 8
    slices of (128 x 8192); every output column block comes from its own
    slice."""
    case = W.AgCase("agb_e4m3_p8_8192x1024x8192", M=8192, N=1024, K=8192, P=8, rank=5, dtype="e4m3",
                    dist="n05", beta=1.0)
    say(f"full: {case.name} generate")
    inp = W.ag_rotb_inputs(case)
    a, bs, c = dev(inp["a"]), [dev(x) for x in inp["b_slices"]], dev(inp["c"])
    kw = dict(M=case.M, N=case.N, K=case.K, rank=case.rank, dtype=tp.E4M3, alpha=case.alpha, beta=case.beta,
              schedule=tp.ROTATE_B)
    d = bf16_empty(case.M, case.N)
    say(f"full: {case.name} staged")
    tp.stage_ag(a, bs, c, d, **kw)
    torch.cuda.synchronize()
    say(f"full: {case.name} oracle")
    ref = oracle.gemm_ag_rotb(inp["a"], inp["b_slices"], inp["c"], case.alpha, case.beta, case.rank, "e4m3", "nk")
    assert_parity(host_f64(d), ref, case.name)
    d2 = bf16_empty(case.M, case.N)
    say(f"full: {case.name} unstaged")
    tp.stage_ag(a, bs, c, d2, flags=tp.UNSTAGED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(d, d2)


def test_full_rs_tileb_bf16():
    """Tiled B at the bf16 reduce-scatter shape: 8 column blocks of 1024 of
    the (8192 x 8192) partial, K = 3584; the incoming partials land on the
    own column block only."""
    case = W.RsCase("rsb_bf16_p8_8192x8192x3584", M=8192, N=8192, K=3584, P=8, rank=6)
    say(f"full: {case.name} generate")
    inp = W.rs_tileb_inputs(case)
    a, b = dev(inp["a"]), dev(inp["b"])
    inc = [dev(x) if x is not None else None for x in inp["incoming"]]
    kw = dict(M=case.M, N=case.N, K=case.K, P=case.P, rank=case.rank, schedule=tp.TILE_B)
    d = bf16_empty(case.M, case.N)
    say(f"full: {case.name} staged")
    tp.stage_rs(a, b, inc, d, **kw)
    torch.cuda.synchronize()
    say(f"full: {case.name} oracle")
    ref = oracle.gemm_rs_tileb(inp["a"], inp["b"], inp["incoming"], 1.0, case.rank, case.P, "nk")
    got = host_f64(d)
    n = case.N // case.P
    own = slice(case.rank * n, (case.rank + 1) * n)
    emitted = np.r_[0:case.rank * n, (case.rank + 1) * n:case.N]
    assert_parity(got[:, emitted], ref[:, emitted], "emitted column blocks")
    assert_parity(got[:, own], ref[:, own], "own column block")
    d2 = bf16_empty(case.M, case.N)
    say(f"full: {case.name} unstaged")
    tp.stage_rs(a, b, inc, d2, flags=tp.UNSTAGED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(d, d2)


WGRAD_FULL = [W.WgCase("wg_x_1024x8192_c8192", M=8192, N=1024, K=8192, P=8, rank=3, gathered="x"),
              W.WgCase("wg_g_w13_4096x3584_c8192", M=8192, N=4096, K=3584, P=8, rank=6, gathered="g")]


@pytest.mark.parametrize("case", WGRAD_FULL, ids=lambda c: c.name)
def test_full_wgrad(case):
    """Weight gradients at full size: of the e4m3 all-gather shape (in bf16, X
    gathered) and of the SwiGLU block's w13 (G = the gathered input), both
    the library's single gathered launch and the staged chain, every output
    element against the oracle."""
    say(f"full: {case.name} generate")
    inp = W.wgrad_inputs(case)
    local, sl = dev(inp["local"]), [dev(x) for x in inp["slices"]]
    g = tp.GATHER_X if case.gathered == "x" else tp.GATHER_G
    say(f"full: {case.name} oracle")
    ref = oracle.wgrad_rows(inp["local"], inp["slices"], case.gathered, list(range(case.N)))
    for groups in (0, 1):
        d = bf16_empty(case.N, case.K)
        say(f"full: {case.name} groups={groups}")
        tp.stage_wgrad(local, sl, d, M=case.M, N=case.N, K=case.K, rank=case.rank, gathered=g, groups=groups)
        torch.cuda.synchronize()
        assert_parity(host_f64(d), ref, f"{case.name}/groups={groups}")


def test_full_qkv():
    """The fused QKV projection at full size (8192 tokens, K = 4096, 512 + 128
    + 128 columns per rank), weights apart, staged and unstaged, every output
    element against the oracle."""
    case = W.QKV
    say(f"full: {case.name} generate")
    inp = W.ag_multi_inputs(case)
    slices = [dev(s) for s in inp["a_slices"]]
    bs = [dev(b) for b in inp["bs"]]
    A = np.concatenate([oracle.decode_bf16(s) for s in inp["a_slices"]], axis=0)
    outs = {}
    for flags in (0, tp.UNSTAGED):
        ds = [bf16_empty(case.M, n) for n in case.ns]
        say(f"full: {case.name} flags={flags}")
        tp.stage_ag_multi(slices, bs, ds, M=case.M, K=case.K, rank=case.rank, flags=flags)
        torch.cuda.synchronize()
        for i, (d, b) in enumerate(zip(ds, inp["bs"])):
            assert_parity(host_f64(d), A @ oracle.decode_bf16(b).T, f"{case.name}/{flags}/out{i}")
        outs[flags] = [d.cpu() for d in ds]
    for x, y in zip(outs[0], outs[tp.UNSTAGED]):
        assert torch.equal(x, y)


def test_full_ffn_backward_one_slot():
    """The FFN backward at the workload size (PB = 4096, L = 8, D = 1280,
    H = 7680): every gradient of one slot against the oracle run on that
    slot alone (the LayerNorm parameter gradients sum over slots and are
    covered at small sizes), with the p04 backward rule for bf16 (per-gradient
    Frobenius relative error <= 2e-2)."""
    case, l = W.C4, 5
    say(f"full: ffn backward generate")
    inp = W.ffn_inputs(case)
    dy = W.ffn_upstream_grad(case)
    t = {k: dev(v) for k, v in inp.items()}
    shapes = dict(dx=(case.PB, case.L, case.D), dw1=(case.L, case.D, 2 * case.H), db1=(case.L, 2 * case.H),
                  dwout=(case.L, case.H, case.D), dbout=(case.L, case.D), dgx=(case.H,), dbx=(case.H,),
                  dgg=(case.H,), dbg=(case.H,))
    grads = {k: bf16_empty(*s) for k, s in shapes.items()}
    say("full: ffn backward run")
    tp.ffn_slot_backward(t["x"], t["w1"], t["b1"], t["wout"], t["gx"], t["bx"], t["gg"], t["bg"], dev(dy), grads,
                         PB=case.PB, L=case.L, D=case.D, H=case.H, eps=case.eps)
    torch.cuda.synchronize()
    say("full: ffn backward oracle (one slot)")
    from oracle import ffn as F
    q = {k: oracle.decode_bf16(inp[k]) for k in ("w1", "b1", "wout", "bout", "gx", "bx", "gg", "bg")}
    q1 = dict(q, w1=q["w1"][l:l + 1], b1=q["b1"][l:l + 1], wout=q["wout"][l:l + 1], bout=q["bout"][l:l + 1])
    X = oracle.decode_bf16(inp["x"][:, l:l + 1])
    ref = F.backward_f64(X, q1, oracle.decode_bf16(dy[:, l:l + 1]), case.eps)
    pairs = dict(dx=(host_f64(grads["dx"])[:, l], ref["x"][:, 0]), dw1=(host_f64(grads["dw1"])[l], ref["w1"][0]),
                 db1=(host_f64(grads["db1"])[l], ref["b1"][0]), dwout=(host_f64(grads["dwout"])[l], ref["wout"][0]),
                 dbout=(host_f64(grads["dbout"])[l], ref["bout"][0]))
    errs = {k: float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-12)) for k, (g, r) in pairs.items()}
    say(f"full: ffn backward slot {l} frobenius {errs}")
    assert all(e <= 2e-2 for e in errs.values()), errs
