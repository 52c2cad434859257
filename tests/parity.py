"""Acceptance check of a bf16 result against the float64 oracle.

Two conditions, both required:
  1. ||gpu - ref||_F / max(||ref||_F, 1e-12) <= 1e-2 (denominator clamp as in
     the p04 statement's backward check, "Cross-node tests and correctness");
  2. every element: |gpu - ref| <= 4 ulp_bf16(max(|ref|, rms(ref))), where
     ulp_bf16(x) = 2^(floor(log2 x) - 7).
"""
import numpy as np

FRO_TOL = 1e-2
ULP_TOL = 4.0


def bf16_ulp(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(x))
    return np.where(x > 0, np.exp2(e - 7.0), 0.0)


def parity_report(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = got - ref
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-12)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    bound = ULP_TOL * bf16_ulp(np.maximum(np.abs(ref), rms))
    bad = ~(np.abs(err) <= bound)           # NaN counts as bad
    worst = float(np.max(np.abs(err) / np.where(bound > 0, bound, 1.0))) if ref.size else 0.0
    return dict(fro=float(fro), n_bad=int(bad.sum()), worst_ulp_ratio=worst, n=int(ref.size))


def assert_parity(got, ref, what=""):
    r = parity_report(got, ref)
    assert r["fro"] <= FRO_TOL and r["n_bad"] == 0, f"{what}: {r}"
    return r
