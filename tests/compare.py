"""Comparators shared by the CPU pins and the GPU parity tests.

Blend + stitch: bit-exact, compared as raw storage bits (so -0 vs +0 and any
NaN payload count as differences).

GroupNorm: compared against the double-precision oracle with the readings of
the stated tolerances:
  fp32 output:       |y - y_ref| <= 1e-5 * max(1, |y_ref|)
  fp16/bf16 output:  |y - y_ref| <= max(1e-2, ulp_T(y_ref))
(a pure relative bound fails near zero outputs; a pure 1e-2 absolute bound
is smaller than one bf16 step once |y| >= 2, so a correctly rounded result
could not meet it).  The count that misses the literal 1e-2 is reported.
"""
from __future__ import annotations

import numpy as np

BITS = {"fp32": np.uint32, "fp16": np.uint16, "bf16": np.uint16}
MANT_BITS = {"fp32": 23, "fp16": 10, "bf16": 7}
MIN_NORMAL_EXP = {"fp32": -126, "fp16": -14, "bf16": -126}


def bits(arr: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(arr)
    return a.view(BITS[dtype]) if a.dtype.itemsize == np.dtype(BITS[dtype]).itemsize else a.astype(BITS[dtype])


def bit_mismatches(got: np.ndarray, want: np.ndarray, dtype: str):
    g, w = bits(got, dtype), bits(want, dtype)
    if g.shape != w.shape:
        raise AssertionError(f"shape mismatch {g.shape} vs {w.shape}")
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    return bad


def assert_bitexact(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    bad = bit_mismatches(got, want, dtype)
    if bad.size:
        g, w = bits(got, dtype).reshape(-1), bits(want, dtype).reshape(-1)
        k = bad[0]
        idx = np.unravel_index(k, got.shape)
        raise AssertionError(f"{what}: {bad.size} of {g.size} elements differ; first at {idx}: "
                             f"got 0x{int(g[k]):x} want 0x{int(w[k]):x}")


def ulp(values: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage type at |values| (binade of each value)."""
    v = np.abs(np.asarray(values, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, MIN_NORMAL_EXP[dtype])
    return np.exp2(e - MANT_BITS[dtype])


def groupnorm_check(got_f64: np.ndarray, ref_f64: np.ndarray, dtype: str):
    """Returns (ok, report dict)."""
    d = np.abs(got_f64 - ref_f64)
    if dtype == "fp32":
        tol = 1e-5 * np.maximum(1.0, np.abs(ref_f64))
    else:
        tol = np.maximum(1e-2, ulp(ref_f64, dtype))
    bad = d > tol
    rep = {
        "max_abs_err": float(d.max()) if d.size else 0.0,
        "n_out_of_tol": int(bad.sum()),
        "n_over_literal": int((d > (1e-5 * np.abs(ref_f64) if dtype == "fp32" else 1e-2)).sum()),
        "n": int(d.size),
    }
    return (not bad.any()) and np.isfinite(got_f64).all(), rep


def ramp_check(got_f64: np.ndarray, ref_f64: np.ndarray, mag_f64: np.ndarray, dtype: str):
    """Normalised-ramp blend against the double oracle.  The kernel sums at
    most 16 weighted terms in fp32 with weights carrying a few roundings each;
    a bound of 2^-18 times the weighted sum of magnitudes covers that with
    room, and a 16-bit output may then round to either neighbour of the exact
    value: one step of the storage type on top.  Returns (ok, report)."""
    d = np.abs(got_f64 - ref_f64)
    tol = 2.0 ** -18 * mag_f64
    if dtype != "fp32":
        tol = tol + ulp(ref_f64, dtype)
    bad = d > tol
    rep = {"max_abs_err": float(d.max()) if d.size else 0.0, "n_out_of_tol": int(bad.sum()),
           "n": int(d.size)}
    return (not bad.any()) and bool(np.isfinite(got_f64).all()), rep
