"""The benchmark's JSON line on the GPU: one short run of the default workload
(a few steps, a short CPU baseline, no extra rows) must print the contract's
fields, a roofline that is its own achieved / peak, and a bit-exact blend and
in-tolerance GroupNorm against the oracle on the same run's output, for the
step and for each of the five workloads' rows."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[bench] short default run", file=sys.stderr, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--flushed-reps", "2", "--no-extra", "--cpu-min-seconds", "0.1",
                        "--cpu-single-seconds", "0", "--probe-reps", "3"], capture_output=True, text=True,
                       timeout=200)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 5 and line["warmup"] == 2
    assert line["unit"] == "GB/s" and line["higher_is_better"] is True and line["dtype"] == "bf16"
    assert line["value"] > 0 and line["ms_per_step"] > 0
    assert "workload" in line["config"]
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert roof["achieved"] == pytest.approx(line["config"]["blend_bytes"] / (roof["launch_us"] * 1e-6) / 1e9)
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert line["parity"]["blend_mismatches"] == 0
    assert line["parity"]["groupnorm_out_of_tol"] == 0
    assert line["parity"]["groupnorm_over_literal_1e-2"] >= 0
    # every workload at full size, in the launch configuration timed, against the oracle
    assert sorted(line["configs"]) == ["1", "2", "3", "4", "5"]
    for k, row in line["configs"].items():
        assert row["blend"]["mismatches"] == 0, k
        assert row["blend"]["frac"] == pytest.approx(row["blend"]["GBps"] / 8000.0)
        assert 0 < row["blend"]["ceiling_us"]
        if "groupnorm" in row:
            assert row["groupnorm"]["out_of_tol"] == 0, k
    assert "groupnorm" in line["configs"]["4"] and "groupnorm" not in line["configs"]["2"]
