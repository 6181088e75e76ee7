"""The blend kernel's fp32 seam coefficients against their definition.

The kernel does not divide in float64: it forms k/e and (e-k)/e from an fp32
reciprocal with one exact-remainder correction (two fused multiply-adds).
tests/csrc/coefficient_check.c restates that arithmetic on the host and
compares it with the weights the diffusers proposal (*Proposed scope*) fixes,
float64 quotients rounded once to fp32, for every (k, e) up to the largest
blend extent the library accepts (4096).  test_oracle_blend.py pins the
oracle's own coefficients against exact rationals.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _run(tmp_path, max_e):
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path / "coefficient_check")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "csrc", "coefficient_check.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe, str(max_e)], capture_output=True, text=True, check=True).stdout.split()
    return {out[i]: int(out[i + 1]) for i in range(0, len(out), 2)}


def test_corrected_reciprocal_equals_float64_weights_up_to_4096(tmp_path):
    got = _run(tmp_path, 4096)
    assert got["pairs"] == 4096 * 4097 // 2
    assert got["wb_mismatches"] == 0 and got["wa_mismatches"] == 0


def test_the_check_sees_a_plain_product():
    """The uncorrected product n * fp32(1/e) is not the float64-rounded weight
    for some (k, e): the correction step is needed, and the check would see
    it dropped."""
    import numpy as np
    bad = 0
    for e in range(1, 600):
        r = np.float32(1.0 / e)
        k = np.arange(e, dtype=np.float32)
        bad += int(np.sum((k * r).astype(np.float32) != (np.arange(e) / e).astype(np.float32)))
    assert bad > 0
