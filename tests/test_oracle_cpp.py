"""The C++17 oracle (oracle/cpp/oracle.cpp) against the numpy oracle, which
the other oracle tests pin to the pages and to the mathematics: the two are
independent writings of the same definitions, so agreement to float64
rounding (different summation orders) on every schedule, layout, element
type and edge case pins the C++ one too. Decoders and permutes must agree
bit for bit."""
import numpy as np
import pytest

import oracle
from oracle import cref
from synth import workloads as W


@pytest.fixture(scope="module", autouse=True)
def built():
    cref.ensure_built()


def close(got, ref):
    assert got.shape == ref.shape
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    scale = max(1.0, float(np.abs(ref[ok]).max())) if ok.any() else 1.0
    assert float(np.abs(got[ok] - ref[ok]).max(initial=0.0)) <= 1e-10 * scale


def test_decoders_every_code():
    e = np.arange(256, dtype=np.uint8)
    got, ref = cref.decode(e, "e4m3"), oracle.decode_e4m3(e)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got, ref = cref.decode(b, "bf16"), oracle.decode_bf16(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])


AG = [c for c in W.SMALL_AG if "medium" not in c.name] + [W.C1]


@pytest.mark.parametrize("case", AG, ids=lambda c: c.name)
def test_gemm_ag(case):
    inp = W.ag_inputs(case)
    for rank in (case.rank, (case.rank + 1) % case.P):
        ref = oracle.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, rank, case.dtype,
                             case.b_layout, swiglu=case.swiglu)
        got = cref.gemm_ag(inp["a_slices"], inp["b"], inp["c"], case.alpha, case.beta, rank, case.dtype,
                           case.b_layout, swiglu=case.swiglu)
        close(got, ref)


RS = [c for c in W.SMALL_RS if "medium" not in c.name] + \
     [W.RsCase("rs_no_incoming", M=4 * 40, N=72, K=64, P=4, rank=1, std=0.5, incoming=False)]


@pytest.mark.parametrize("case", RS, ids=lambda c: c.name)
def test_gemm_rs(case):
    inp = W.rs_inputs(case)
    inc = inp["incoming"] if case.incoming else None
    ref = oracle.gemm_rs(inp["a"], inp["b"], inc, case.alpha, case.rank, case.P, case.b_layout)
    got = cref.gemm_rs(inp["a"], inp["b"], inc, case.alpha, case.rank, case.P, case.b_layout)
    close(got, ref)


@pytest.mark.parametrize("case", [c for c in W.SMALL_AG_ROTB if "medium" not in c.name], ids=lambda c: c.name)
def test_gemm_ag_rotb(case):
    inp = W.ag_rotb_inputs(case)
    ref = oracle.gemm_ag_rotb(inp["a"], inp["b_slices"], inp["c"], case.alpha, case.beta, case.rank, case.dtype,
                              case.b_layout)
    got = cref.gemm_ag_rotb(inp["a"], inp["b_slices"], inp["c"], case.alpha, case.beta, case.rank, case.dtype,
                            case.b_layout)
    close(got, ref)


@pytest.mark.parametrize("case", W.SMALL_RS_TILEB, ids=lambda c: c.name)
def test_gemm_rs_tileb(case):
    inp = W.rs_tileb_inputs(case)
    ref = oracle.gemm_rs_tileb(inp["a"], inp["b"], inp["incoming"], case.alpha, case.rank, case.P, case.b_layout)
    got = cref.gemm_rs_tileb(inp["a"], inp["b"], inp["incoming"], case.alpha, case.rank, case.P, case.b_layout)
    close(got, ref)


@pytest.mark.parametrize("case", W.SMALL_FFN, ids=lambda c: c.name)
def test_ffn_slot_forward(case):
    inp = W.ffn_inputs(case)
    close(cref.ffn_slot_forward(inp, case.eps), oracle.ffn_slot_forward(inp, case.eps))


@pytest.mark.parametrize("case", W.SMALL_SWIGLU, ids=lambda c: c.name)
def test_swiglu_hidden(case):
    inp = W.swiglu_inputs(case)
    close(cref.swiglu_hidden(inp["x_shards"], inp["w13"]), oracle.swiglu_hidden(inp["x_shards"], inp["w13"]))


@pytest.mark.parametrize("P,B,T,D,dt", [(2, 1, 2, 1, np.uint16), (4, 3, 8, 5, np.uint16), (8, 2, 16, 3, np.uint8)])
def test_permutes_bit_exact(P, B, T, D, dt):
    rng = np.random.default_rng(7)
    xs = [rng.integers(0, 200, (B, T, D)).astype(dt) for _ in range(P)]
    for r in range(P):
        assert np.array_equal(cref.dispatch(xs, r), oracle.dispatch(xs, r))
    ys = [rng.integers(0, 200, (P * B, T // P, D)).astype(dt) for _ in range(P)]
    for r in range(P):
        assert np.array_equal(cref.combine(ys, r), oracle.combine(ys, r))
