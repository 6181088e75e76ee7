"""The benchmark's host-side contract, on the CPU: it refuses more than one
GPU with a message, reports a missing GPU instead of falling back, and its
algorithmic byte count of the normalised-ramp blend equals a brute-force count
of the tile positions that carry weight."""
from __future__ import annotations

import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = _run("--gpus", str(n))
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == n


def test_no_gpu_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible here")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "no GPU" in r.stdout


def _weighted_positions(origins, extents, m, r):
    """Brute force along one axis: per tile, the positions whose ramp factor is
    above zero (a tile weighs nothing within the margin of an edge it shares)."""
    n = len(origins)
    count = 0
    for k, (o, s) in enumerate(zip(origins, extents)):
        p = np.arange(o, o + s)
        f = np.ones(s)
        if k > 0:
            f *= np.clip((p - o - m) / r, 0, 1)
        if k < n - 1:
            f *= np.clip((o + s - 1 - p - m) / r, 0, 1)
        count += int((f > 0).sum())
    return count


@pytest.mark.parametrize("name", sorted(workloads.RAMP_WORKLOADS))
def test_ramp_bytes_equal_a_brute_force_count(name):
    bench = _bench_module()
    w = workloads.RAMP_WORKLOADS[name]
    ch = _weighted_positions(w.origins_h, w.extents_h, w.margin[0], w.ramp[0])
    cw = _weighted_positions(w.origins_w, w.extents_w, w.margin[1], w.ramp[1])
    planes = int(np.prod(w.lead))
    LH, LW = w.out_shape[-2:]
    assert bench.ramp_bytes(w, 2) == planes * (ch * cw + LH * LW) * 2
