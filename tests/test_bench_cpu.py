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


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size_X,Grid_Size_Y,Counter_Name,Counter_Value\n")
        for r in rows:
            f.write(",".join(str(v) for v in r) + "\n")


def test_traffic_record_from_counter_runs(tmp_path):
    """Dispatches grouped by (kernel, grid) in launch order, averaged per
    dispatch, scaled by the 256 MiB copy, and matched to the launches of one
    profile mode of the benchmark; the file records the sources' hashes and
    keeps the records of other modes."""
    from benchkit import traffic
    cfg = workloads.CONFIGS[4]
    kernels = [("sb::blend_stitch_kernel", 1), ("sb::gn_stats_kernel", 2), ("sb::gn_norm_kernel", 3)]
    for counter, scale in (("FETCH_SIZE", 0.5), ("WRITE_SIZE", 1.0)):
        rows, d = [], 0
        for name, grid in kernels:  # each call's launches together, as the profile mode makes them
            for rep in range(2):  # two dispatches of every launch, values 100 and 300 KiB
                d += 1
                # a counter split over two instances of the same dispatch is summed
                rows += [(d, name, grid, 1, counter, (100 + 200 * rep) / 2),
                         (d, name, grid, 1, counter, (100 + 200 * rep) / 2)]
        d += 1
        rows.append((d, "__amd_rocclr_copyBuffer", 99, 1, counter, 262144 * scale))
        rows.append((d + 1, "torch_fill", 7, 1, counter, 5.0))
        _counter_csv(str(tmp_path / counter / "run" / "run_counter_collection.csv"), rows)
    out = tmp_path / "traffic.json"
    json.dump({"launches": {"ramp:other": {"kept": True}}}, open(out, "w"))
    traffic.write_traffic(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"), "config4", path=str(out))
    rec = json.load(open(out))
    assert rec["launches"]["ramp:other"] == {"kept": True}
    blend = rec["launches"]["config4-blend"]
    assert blend["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert blend["calibration"]["write_scale"] == pytest.approx(1.0)
    assert [n for n in rec["launches"] if n.startswith("config4")] == [
        "config4-blend", "config4-gn-stats", "config4-gn-norm"]
    assert blend["dispatches"] == 2
    assert blend["fetch_kib_per_dispatch"] == pytest.approx(200.0)
    assert blend["hbm_bytes_per_launch"] == pytest.approx(200 * 1024 * 2.0 + 200 * 1024)
    w = cfg.blend
    out_elems = w.N * w.C * 49 * 480 * 832
    assert blend["algorithmic_bytes_per_launch"] == (w.tile_elems() + out_elems) * 2
    gn = cfg.groupnorm
    assert rec["launches"]["config4-gn-norm"]["algorithmic_bytes_per_launch"] == 2 * 2 * int(np.prod(gn.shape))
    for name, r in rec["launches"].items():
        if name.startswith("config4"):
            for f, h in r["sources_sha256"].items():
                assert os.path.exists(os.path.join(ROOT, f)) and len(h) == 64
    # the readable table: one row per launch with the scaled bytes and the excess
    rec["launches"].pop("ramp:other")
    json.dump(rec, open(out, "w"))
    md = traffic.traffic_table(str(out))
    assert md.count("| config4-") == 3
    assert f"| {blend['hbm_bytes_per_launch']:.0f} | {blend['algorithmic_bytes_per_launch']} |" in md
    assert "--pmc FETCH_SIZE" in md and "benchkit.traffic traffic <w>" in md


def test_kernel_trace_summary(tmp_path):
    """Per (kernel, grid): dispatch count and average / min / max duration."""
    from benchkit import traffic
    d = tmp_path / "kt" / "run"
    os.makedirs(d)
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Start_Timestamp,End_Timestamp\n")
        f.write("sb::a,10,1,1,1000,3000\n" "sb::b,5,1,1,4000,5000\n" "sb::a,10,1,1,6000,10000\n")
    md = traffic.summarize_trace(str(tmp_path / "kt"), "t", "cmd")
    assert "| `sb::a` | 10x1x1 | 2 | 3.00 | 2.00 | 4.00 |" in md
    assert "| `sb::b` | 5x1x1 | 1 | 1.00 | 1.00 | 1.00 |" in md


def test_probe_library_checks_its_arguments_on_host():
    """The streaming probe refuses bad sizes and pointers before any launch."""
    import ctypes

    import benchkit
    if not os.path.exists(benchkit.LIB):
        pytest.skip("probe library not built")
    L = benchkit.lib()
    f = L.benchkit_stream
    assert f(None, 1024, None, 0, 0x1000, 4, 0, 0, None) == -1          # null source
    assert f(0x10000, 1000, None, 0, 0x1000, 4, 0, 0, None) == -1       # not a multiple of 16
    assert f(0x10000, 1024, None, 512, 0x1000, 4, 0, 0, None) == -1     # writes without a destination
    assert f(0x10000, 1024, 0x20000, 2048, 0x1000, 4, 0, 0, None) == -1  # writes more than it reads
    assert f(0x10000, 1024, 0x20008, 512, 0x1000, 4, 0, 0, None) == -1  # misaligned destination
    assert f(0x10000, 1024, None, 0, 0x1000, 3, 0, 0, None) == -1       # no such shape
    assert f(0x10000, 16 << 32, None, 0, 0x1000, 1, 0, 0, None) == -1   # grid beyond 2^32 work-items
    del ctypes
