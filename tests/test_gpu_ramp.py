"""GPU parity of the normalised-ramp blend of wide tiles against the double
oracle, within the tolerance derived in compare.ramp_check; positions where a
single tile carries weight must equal that tile exactly."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import compare
import oracle
import workloads as W
from gpu_util import as_f64, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import seam_blending_patch_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_grid(w, tiles, misalign=False):
    nh, nw = len(w.origins_h), len(w.origins_w)
    grid, k = [], 0
    for i in range(nh):
        row = []
        for j in range(nw):
            t = to_dev(tiles[k], w.dtype)
            if misalign:
                buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
                v = buf[1:].view(t.shape)
                v.copy_(t)
                t = v
            row.append(t)
            k += 1
        grid.append(row)
    return grid


def single_tile_mask(w):
    """(rows, cols) boolean masks of positions where one tile has weight."""
    def axis(origins, extents, m):
        L = max(o + e for o, e in zip(origins, extents))
        cnt = np.zeros(L, int)
        n = len(origins)
        for k, (o, e) in enumerate(zip(origins, extents)):
            lo = o + m + 1 if k > 0 else o
            hi = o + e - 1 - m if k < n - 1 else o + e
            cnt[lo:max(lo, hi)] += 1
        return cnt == 1
    return axis(w.origins_h, w.extents_h, w.margin[0]), axis(w.origins_w, w.extents_w, w.margin[1])


def check(sb, w, what="", misalign=False, out=None):
    _say(f"[ramp] {what} {w.name} {w.dtype} lead={tuple(w.lead)} tiles={len(w.origins_h)}x{len(w.origins_w)}"
         f" out={w.out_shape} misalign={misalign}")
    tiles = W.draw_ramp_tiles(w)
    y = sb.vae_tile_ramp_blend(dev_grid(w, tiles, misalign), w.origins_h, w.origins_w, w.margin,
                               w.ramp, out=out)
    torch.cuda.synchronize()
    got = as_f64(from_dev(y, w.dtype), w.dtype)
    ref, mag = oracle.ramp_blend(tiles, w.lead, w.origins_h, w.extents_h, w.origins_w, w.extents_w,
                                 w.margin, w.ramp, w.dtype, with_magnitude=True)
    ok, rep = compare.ramp_check(got, ref, mag, w.dtype)
    _say(f"      {rep}")
    assert ok, f"{what} {w.name}: {rep}"
    rows, cols = single_tile_mask(w)
    sel = (slice(None),) * len(w.lead) + np.ix_(rows, cols)
    assert np.array_equal(got[sel], ref[sel]), "single-tile positions must be exact copies"
    return y


def test_more_planes_than_one_launch_holds(sb):
    # 2^24 + 3 planes of one 1x2 tile: more blocks than a grid's x extent
    # takes, so the planes go in two launches
    check(sb, RW("planes", "bf16", (1, (1 << 24) + 3), [0], [1], [0], [2], (4, 4), (8, 8), seed=5,
                 clamp=None), "planes")


def test_tall_canvas_of_many_row_bands(sb):
    # a 310,000-row canvas two vectors wide: about 1,200 row bands of a few
    # hundred rows over three row segments, two of them single-tile
    check(sb, RW("tall", "bf16", (1, 1), [0, 150000], [160000, 160000], [0], [16], (4, 4), (8, 8), seed=6),
          "bands across launches")


@pytest.mark.parametrize("name", sorted(W.RAMP_WORKLOADS))
def test_named_workloads_full_size(sb, name):
    check(sb, W.RAMP_WORKLOADS[name], "workload")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_random_layouts(sb, dtype):
    for seed in range(24):
        align = 4 if dtype == "fp32" else 8
        w = W.random_ramp_workload(100 + seed, dtype, lead=(1, 2) if seed % 3 else (2, 1, 3),
                                   align=align if seed % 2 else 1)
        check(sb, w, f"random {seed}", misalign=(seed % 5 == 4))


RW = W.RampWorkload
EDGE = [
    RW("single-tile", "bf16", (1, 2), [0], [37], [0], [64], (4, 4), (8, 8), seed=1, clamp=None),
    RW("three-with-weight", "fp16", (1, 2), [0, 6, 12], [30] * 3, [0, 8, 16], [40] * 3, (2, 2), (6, 6),
       seed=2, clamp=None),
    RW("four-with-weight", "fp32", (1, 1), [0, 4, 8, 12], [30] * 4, [0, 4, 8, 12], [40] * 4, (0, 0),
       (9, 9), seed=3, clamp=None),
    RW("48x48-tiles", "bf16", (1, 1), [k * 24 for k in range(48)], [40] * 48, [k * 32 for k in range(48)],
       [48] * 48, (3, 3), (5, 5), seed=4, clamp=None),
    RW("wide-canvas", "bf16", (1, 1), [0, 16], [32, 32], [0, 300000], [320000, 320000], (4, 4), (8, 8),
       seed=5, clamp=None),
    RW("uneven-extents", "fp16", (2, 3), [0, 100, 150], [120, 90, 60], [0, 64, 200], [96, 160, 64],
       (5, 5), (10, 10), seed=6, clamp=None),
    RW("margin-0-ramp-1", "bf16", (1, 1), [0, 10], [20, 20], [0, 8], [16, 16], (0, 0), (1, 1), seed=7,
       clamp=None),
]


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_edge_layouts(sb, w):
    check(sb, w, "edge")
    if w.dtype != "fp32":
        check(sb, w, "edge", misalign=True)


def test_empty_batch_and_bad_layouts(sb):
    t = torch.zeros((0, 3, 32, 32), dtype=torch.bfloat16, device="cuda")
    y = sb.vae_tile_ramp_blend([[t, t], [t, t]], [0, 16], [0, 16], 4, 8)
    assert y.shape == (0, 3, 48, 48)
    a = torch.zeros((1, 1, 20, 20), device="cuda")
    with pytest.raises(sb.SeamBlendError) as ei:  # an overlap of 9 leaves a position uncovered
        sb.vae_tile_ramp_blend([[a, a]], [0], [0, 11], 4, 8)
    assert ei.value.code == -2
    with pytest.raises(sb.SeamBlendError):  # origins must increase
        sb.vae_tile_ramp_blend([[a, a]], [0], [0, 0], 4, 8)


def test_output_buffer_and_graph_replay(sb):
    w = W.RAMP_WORKLOADS["flux-1600-bf16"]
    tiles = W.draw_ramp_tiles(w)
    grid = dev_grid(w, tiles)
    out = torch.full(w.out_shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    plan = sb.RampBlend(grid, w.origins_h, w.origins_w, w.margin, w.ramp, out=out)
    eager = plan().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        plan()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            plan()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        for row in grid:  # new inputs between replays
            for t in row:
                t.mul_(-1)
        torch.cuda.synchronize()
        eager = plan().clone()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


# Qwen-Image-2.1 (16x) at the sizes of the pages' real-weight checks, in the
# 32-latent floor tiles placed by the library's planner, and FLUX.1 (8x) at
# 1600 px in the fewest-calls tiles: planner and blend together, against the
# oracle's layout and the oracle's blend
PAGES_SIZES = [((1024, 1024), 16, "edge_aligned", [32, 16]),
               ((1344, 1344), 16, "edge_aligned", [32, 16]),
               ((1536, 2752), 16, "edge_aligned", [32, 16]),
               ((864, 1184), 16, "edge_aligned", [32, 16]),
               ((2048, 2048), 16, "edge_aligned", [32, 16]),
               ((1600, 1600), 8, "fewest_calls", [128, 96, 32, 128])]


@pytest.mark.parametrize("size,ratio,rule,params", PAGES_SIZES, ids=lambda v: str(v))
def test_planner_layouts_blend_at_the_pages_sizes(sb, size, ratio, rule, params):
    from oracle import layout as ol
    axes = []
    for px in size:
        L = px // ratio
        o, e = sb.vae_tile_layout(L, rule, params)
        assert list(zip(o, e)) == ol.layout(L, rule, params)
        axes.append(([v * ratio for v in o], [v * ratio for v in e]))
    (oh, eh), (ow, ew) = axes
    w = W.RampWorkload(f"pages-{size[0]}x{size[1]}", "bf16", (1, 3), oh, eh, ow, ew, (4 * ratio,) * 2,
                       (8 * ratio,) * 2, seed=size[0] + size[1])
    assert w.out_shape[-2:] == tuple(size)
    check(sb, w, "planner+blend")


def test_deterministic_and_concurrent(sb):
    # two runs give identical bits; two layouts on two streams at once give the
    # serial results
    plans, serial = [], []
    for name in ("qwen21-2048-bf16", "flux-1600-bf16"):
        w = W.RAMP_WORKLOADS[name]
        grid = dev_grid(w, W.draw_ramp_tiles(w))
        p = sb.RampBlend(grid, w.origins_h, w.origins_w, w.margin, w.ramp)
        a = p().clone()
        b = p().clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        plans.append((p, grid))
        serial.append(a)
    for p, _ in plans:
        p.out.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (p, _), st in zip(plans, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for _ in range(3):
                p()
    torch.cuda.synchronize()
    for (p, _), want in zip(plans, serial):
        assert torch.equal(p.out.view(torch.int16), want.view(torch.int16))
