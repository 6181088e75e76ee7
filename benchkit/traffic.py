"""Readers of rocprofv3 output for the benchmark.

HBM traffic per launch (``profiles/traffic.json``) from two ``--pmc`` runs of
one profile mode of ``bench.py`` (``FETCH_SIZE``, then ``WRITE_SIZE``; KiB per
dispatch): dispatches are grouped by (kernel, grid) in launch order, averaged
per dispatch, matched in order to the library launches that mode makes, and
scaled by what the same counter reads for the plain 256 MiB device copy the
profile modes run (``__amd_rocclr_copyBuffer``).  Each record keeps the
SHA-256 of the sources it was taken on, so the benchmark reports it only while
they are unchanged.

Kernel-time summaries (``profiles/*.md``) from a ``--kernel-trace`` run:
dispatches grouped by (kernel, grid), with count and average / min / max
duration.

    python -m benchkit.traffic traffic {config1..config5|extra} FETCH_DIR WRITE_DIR
    python -m benchkit.traffic trace TRACE_DIR OUT.md "TITLE" "COMMAND"
    python -m benchkit.traffic table OUT.md
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

KERNEL_SOURCES = {
    "blend": ["seam_blending_patch_amd/csrc/blend_stitch.hip", "seam_blending_patch_amd/csrc/abi.cpp"],
    "gn": ["seam_blending_patch_amd/csrc/groupnorm.hip", "seam_blending_patch_amd/csrc/abi.cpp"],
    "ramp": ["seam_blending_patch_amd/csrc/ramp_blend.hip", "seam_blending_patch_amd/csrc/ramp.cpp"],
}
COMMON_SOURCES = ["seam_blending_patch_amd/csrc/sb_internal.h", "seam_blending_patch_amd/csrc/sb_vec.h"]
RAMP_NAMES = ("qwen21-2048-bf16", "qwen21-2752x1536-bf16", "flux-1600-bf16", "qwen21-encode-2048-bf16")
CAL_BYTES = 256 << 20


def ramp_bytes(w, elem):
    """Algorithmic bytes of one normalised-ramp blend: every tile position with
    weight read once (a tile weighs nothing within the margin of a shared edge,
    so those positions are never needed) and every output position written once."""
    def counts(origins, extents, m):
        n, c = len(origins), []
        for k, (o, e) in enumerate(zip(origins, extents)):
            lo = o + m + 1 if k > 0 else o
            hi = o + e - 1 - m if k < n - 1 else o + e
            c.append(max(0, hi - lo))
        return c
    ch = counts(w.origins_h, w.extents_h, w.margin[0])
    cw = counts(w.origins_w, w.extents_w, w.margin[1])
    planes = 1
    for v in w.lead:
        planes *= v
    LH, LW = w.out_shape[-2:]
    return planes * (sum(ch) * sum(cw) + LH * LW) * elem


def blend_out_elems(w):
    """Output elements of a stock blend + stitch: per axis (n - 1) * R + last extent."""
    L = [(len(e) - 1) * r + e[-1] for e, r in zip((w.ext_t, w.ext_h, w.ext_w), w.row_limit)]
    return w.N * w.C * L[0] * L[1] * L[2]


def blend_bytes(w):
    import workloads
    return (w.tile_elems() + blend_out_elems(w)) * workloads.ITEMSIZE[w.dtype]


def launch_names(what):
    """(name, part, algorithmic bytes) of the library launches a profile mode
    of bench.py makes, in launch order."""
    import numpy as np

    import workloads
    if what == "extra":
        out = []
        for name in RAMP_NAMES:
            rw = workloads.RAMP_WORKLOADS[name]
            out.append(("ramp:" + name, "ramp", ramp_bytes(rw, workloads.ITEMSIZE[rw.dtype])))
        for name, ew in workloads.ENCODE_BLEND_WORKLOADS.items():
            out.append(("encode-blend:" + name, "blend", blend_bytes(ew)))
        return out
    k = int(what.replace("config", ""))
    cfg = workloads.CONFIGS[k]
    out = [(f"config{k}-blend", "blend", blend_bytes(cfg.blend))]
    if cfg.groupnorm is not None:
        n = int(np.prod(cfg.groupnorm.shape)) * workloads.ITEMSIZE[cfg.groupnorm.dtype]
        out += [(f"config{k}-gn-stats", "gn", n), (f"config{k}-gn-norm", "gn", 2 * n)]
    return out


def read_groups(d):
    """[((kernel, grid), average counter value per dispatch, dispatches)] of
    the one counter_collection.csv under d, in order of first dispatch."""
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(paths) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {paths}")
    order, vals = [], {}
    rows = sorted(csv.DictReader(open(paths[0])), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        gk = tuple(r[k] for k in sorted(r) if k.startswith("Grid_Size"))
        key = (r["Kernel_Name"], gk)
        if key not in vals:
            order.append(key)
            vals[key] = {}
        vals[key][r["Dispatch_Id"]] = vals[key].get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return [(k, sum(vals[k].values()) / len(vals[k]), len(vals[k])) for k in order]


def _sha(f):
    return hashlib.sha256(open(os.path.join(ROOT, f), "rb").read()).hexdigest()


def write_traffic(fetch_dir, write_dir, what, path=None, command=None):
    """Merge the records of one profile mode into traffic.json; returns its path."""
    def split(gs):
        ours = [g for g in gs if "sb::" in g[0][0]]
        copy = [g for g in gs if "copyBuffer" in g[0][0]]
        if not copy:
            raise SystemExit("no device copy kernel in the counter run (the profile modes run one)")
        return ours, max(copy, key=lambda g: g[1])

    fo, fc = split(read_groups(fetch_dir))
    wo, wc = split(read_groups(write_dir))
    fscale, wscale = CAL_BYTES / (fc[1] * 1024), CAL_BYTES / (wc[1] * 1024)
    names = launch_names(what)
    if len(fo) != len(names) or len(wo) != len(names) or [g[0] for g in fo] != [g[0] for g in wo]:
        raise SystemExit(f"{len(fo)} / {len(wo)} launch groups in the counter runs, {len(names)} expected")
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec["what"] = ("HBM bytes per launch from rocprofv3 PMC counters FETCH_SIZE and WRITE_SIZE (KiB per "
                   "dispatch), each scaled by what the counter reads for a plain 256 MiB device copy "
                   "(__amd_rocclr_copyBuffer) in the same run")
    rec.pop("calibration", None)
    rec.pop("commands", None)
    launches = rec.setdefault("launches", {})
    for (name, part, alg), f, w in zip(names, fo, wo):
        hbm = f[1] * 1024 * fscale + w[1] * 1024 * wscale
        launches[name] = {"kernel": f[0][0], "grid": list(f[0][1]), "dispatches": f[2],
                          "sources_sha256": {s: _sha(s) for s in KERNEL_SOURCES[part] + COMMON_SOURCES},
                          "fetch_kib_per_dispatch": f[1], "write_kib_per_dispatch": w[1],
                          "calibration": {"bytes": CAL_BYTES, "fetch_kib": fc[1], "write_kib": wc[1],
                                          "fetch_scale": fscale, "write_scale": wscale},
                          "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg,
                          "excess": hbm / alg - 1.0,
                          "command": command or f"bench.py --profile {what}"}
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    for name, _, _ in names:
        r = launches[name]
        print(f"{name:40s} {r['hbm_bytes_per_launch']:14.0f} B  algorithmic {r['algorithmic_bytes_per_launch']:12d}"
              f"  {100 * r['excess']:+.1f}%  ({r['kernel'][:48]})")
    return path


def summarize_trace(trace_dir, title, command):
    """Markdown table of a --kernel-trace run: per (kernel, grid), dispatches
    and average / min / max duration in microseconds."""
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if len(paths) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {trace_dir}, found {paths}")
    groups, order = {}, []
    for r in csv.DictReader(open(paths[0])):
        grid = tuple(int(r[k]) for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z") if k in r)
        key = (r["Kernel_Name"], grid)
        if key not in groups:
            order.append(key)
            groups[key] = []
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```",
             "cd /tmp && export TMPDIR=/tmp", command, "```", "",
             "| kernel | grid | dispatches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for key in order:
        d = groups[key]
        name = key[0] if len(key[0]) <= 90 else key[0][:87] + "..."
        lines.append(f"| `{name}` | {'x'.join(map(str, key[1]))} | {len(d)} | {sum(d) / len(d):.2f} | "
                     f"{min(d):.2f} | {max(d):.2f} |")
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        lines += ["", "rocprofv3 --stats (per kernel name, all grids together):", "",
                  "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        for r in csv.DictReader(open(stats[0])):
            name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
            lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(lines) + "\n"


def pmc_command(what, fetch_dir=None, write_dir=None):
    """The commands that make one profile mode's traffic records, with the
    counter runs' output directories as given (placeholders when none)."""
    fetch_dir = fetch_dir or f"<out>/pmc_FETCH_SIZE_{what}"
    write_dir = write_dir or f"<out>/pmc_WRITE_SIZE_{what}"
    return (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
            f"python3 bench.py --profile {what} --steps 3 --warmup 1; the same with WRITE_SIZE into "
            f"{write_dir}; python3 -m benchkit.traffic traffic {what} {fetch_dir} {write_dir}")


def traffic_table(path=None):
    """Markdown table of traffic.json: per launch, counted HBM bytes against
    the algorithmic bytes, with the counter readings and copy calibration."""
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path))
    lines = ["# HBM traffic per launch (rocprofv3 PMC FETCH_SIZE, WRITE_SIZE)", "", rec["what"] + ".", "",
             "Commands (from the repository root, on one MI355X, one counter per run, each under "
             "`timeout -s KILL 120`), for each profile mode `<w>` of config1..config5 and extra:", "", "```",
             "cd /tmp && export TMPDIR=/tmp", pmc_command("<w>"), "```", "",
             "| launch | kernel | fetch KiB | write KiB | fetch scale | HBM bytes | algorithmic bytes | excess |",
             "|---|---|---|---|---|---|---|---|"]
    for name, r in rec["launches"].items():
        k = r["kernel"] if len(r["kernel"]) <= 60 else r["kernel"][:57] + "..."
        lines.append(f"| {name} | `{k}` | {r['fetch_kib_per_dispatch']:.1f} | {r['write_kib_per_dispatch']:.1f} | "
                     f"{r['calibration']['fetch_scale']:.3f} | {r['hbm_bytes_per_launch']:.0f} | "
                     f"{r['algorithmic_bytes_per_launch']} | {100 * r['excess']:+.1f}% |")
    return "\n".join(lines) + "\n"


def main(argv):
    if len(argv) >= 4 and argv[0] == "traffic":
        write_traffic(argv[2], argv[3], argv[1], command=pmc_command(argv[1], argv[2], argv[3]))
    elif len(argv) >= 2 and argv[0] == "table":
        md = traffic_table()
        with open(argv[1], "w") as f:
            f.write(md)
        print(md)
    elif len(argv) >= 5 and argv[0] == "trace":
        md = summarize_trace(argv[1], argv[3], argv[4])
        with open(argv[2], "w") as f:
            f.write(md)
        print(md)
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
