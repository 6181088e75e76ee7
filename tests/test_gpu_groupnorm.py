"""GPU parity of the two-pass patch GroupNorm against the double-precision CPU
oracle (unsplit GroupNorm), within the stated tolerances read as
  fp32: |y - y_ref| <= 1e-5 * max(1, |y_ref|)
  fp16 / bf16: |y - y_ref| <= max(1e-2, one step of the output type at y_ref),
plus the per-patch statistics against the oracle's double per-patch ones."""
from __future__ import annotations

import dataclasses

import sys

import numpy as np
import pytest
import torch

import compare
import oracle
import workloads
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


def run(sb, gw, x, g, b, stats=False, out=None, x_dev=None):
    xd = x_dev if x_dev is not None else to_dev(x, gw.dtype)
    gd = None if g is None else to_dev(g, gw.dtype)
    bd = None if b is None else to_dev(b, gw.dtype)
    ps = None
    if stats:
        ps = torch.full((gw.shape[0], gw.groups, gw.n_patches, 3), float("nan"), device="cuda")
    y = sb.patch_groupnorm(xd, gw.groups, gw.split_axis, gw.n_patches, gw.eps, gd, bd,
                           out=out, patch_stats=ps)
    torch.cuda.synchronize()
    return y, ps


def check(sb, gw, x, g, b, what=""):
    _say(f"[gn] {what} {gw.name} shape={tuple(gw.shape)} P={gw.n_patches} axis={gw.split_axis} {gw.dtype}")
    y, ps = run(sb, gw, x, g, b, stats=True)
    ref, mean, var = oracle.groupnorm(x, gw.groups, gw.eps, g, b, gw.dtype)
    ok, rep = compare.groupnorm_check(as_f64(from_dev(y, gw.dtype), gw.dtype), ref, gw.dtype)
    _say(f"      {rep}")
    assert ok, f"{what} {gw.name}: {rep}"
    st = oracle.patch_stats(x, gw.groups, gw.split_axis, gw.n_patches, gw.dtype)
    got = ps.cpu().numpy().astype(np.float64)
    assert np.array_equal(got[..., 0], st[..., 0]), "per-patch counts"
    scale = np.maximum(1.0, np.abs(st[..., 1]))
    assert np.all(np.abs(got[..., 1] - st[..., 1]) <= 2e-5 * scale), "per-patch means"
    assert np.all(np.abs(got[..., 2] - st[..., 2]) <= 1e-4 * np.maximum(st[..., 2], 1.0)), "per-patch M2"
    return y, rep


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_config_full_size(sb, cfg):
    gw, (x, g, b) = workloads.draw_config_groupnorm(cfg)
    check(sb, gw, x, g, b, f"config {cfg}")


@pytest.mark.parametrize("cfg,dtype", [(3, "fp16"), (3, "fp32"), (4, "fp16"), (4, "fp32")])
def test_config_shapes_in_other_dtypes(sb, cfg, dtype):
    # the workloads' activation shapes, patch splits and offsets at full size
    # in dtypes they are not specified in, at that dtype's tolerance
    base = workloads.CONFIGS[cfg].groupnorm
    gw = dataclasses.replace(base, name=f"{base.name}-as-{dtype}", dtype=dtype, seed=60 + cfg)
    x, g, b = workloads.draw_groupnorm(gw)
    check(sb, gw, x, g, b, f"config {cfg} shape")


def _gw(shape, dtype, G, axis, P, seed, affine=True, offset=("uniform", -2.0, 2.0)):
    return workloads.GroupNormWorkload("rand", dtype, shape, G, axis, P, 1e-6, seed, offset=offset,
                                       affine=affine)


CASES = [
    ((2, 8, 16, 24), 4, 2, 3),
    ((1, 32, 33, 40), 8, 3, 5),      # ragged patches along W
    ((3, 6, 7, 9), 3, 2, 4),         # tiny, scalar path
    ((1, 16, 5, 12, 16), 4, 2, 2),   # split along T
    ((1, 16, 5, 12, 16), 4, 3, 4),   # split along H (5-D)
    ((1, 16, 5, 12, 16), 4, 4, 8),   # split along W (5-D)
    ((2, 12, 6, 10), 3, 2, 9),       # more patches than rows: empty patches
    ((1, 8, 64, 64), 2, 3, 64),      # the maximum patch count
    ((2, 4, 100), 2, 2, 3),          # 3-D
    ((1, 64, 40, 40), 32, 2, 1),     # a single patch
    ((1, 8192, 16, 16), 64, 2, 3),   # 8192 (n, c) planes of one normalise block each
    ((1, 8, 6, 5), 2, 3, 9),         # W split, more patches than columns: empty patches
    ((1, 4, 3, 4096), 2, 3, 4),      # W split, rows of 512-1024 vectors
    ((1, 4, 3, 8192), 2, 3, 3),      # W split, ragged, rows wider than one block: patch-run path
]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_random_shapes(sb, dtype):
    for k, (shape, G, axis, P) in enumerate(CASES):
        gw = _gw(shape, dtype, G, axis, P, seed=50 + k, affine=(k % 3 != 2))
        x, g, b = workloads.draw_groupnorm(gw)
        check(sb, gw, x, g, b, f"case {k}")


def _random_case(rng):
    # a random activation: 3-D to 5-D, 1-32 groups of 1-8 channels, split
    # along any spatial axis into 1 to a few more patches than positions
    ndim = int(rng.integers(3, 6))
    N = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    C = G * int(rng.choice([1, 2, 3, 4, 8]))
    hi = {3: 400, 4: 64, 5: 24}[ndim]
    spatial = [int(rng.integers(1, hi + 1)) for _ in range(ndim - 2)]
    axis = int(rng.integers(2, ndim))
    L = spatial[axis - 2]
    P = int(rng.integers(1, min(64, L + 2) + 1))
    return (N, C, *spatial), G, axis, P


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_random_activations_many_seeds(sb, dtype):
    # 60 random shapes per dtype: every patch layout the host can pick (patch
    # runs, whole-row blocks, empty patches), vector and scalar paths, with and
    # without affine and per-patch offsets; fp32 at the 1e-5 reading
    rng = np.random.default_rng(77 if dtype == "fp32" else 78)
    for k in range(60):
        shape, G, axis, P = _random_case(rng)
        offset = ("uniform", -2.0, 2.0) if k % 2 == 0 else None
        gw = _gw(shape, dtype, G, axis, P, seed=700 + k, affine=(k % 3 != 1), offset=offset)
        x, g, b = workloads.draw_groupnorm(gw)
        check(sb, gw, x, g, b, f"random {k}")


def test_constant_group_gives_beta_exactly(sb):
    gw = _gw((1, 16, 8, 8), "fp32", 4, 2, 2, seed=1, offset=None)
    x = np.full(gw.shape, 2.5, np.float32)
    g = np.linspace(0.5, 1.5, 16).astype(np.float32)
    b = np.linspace(-1, 1, 16).astype(np.float32)
    y, _ = run(sb, gw, x, g, b)
    want = np.broadcast_to(b[None, :, None, None], gw.shape)
    assert np.array_equal(from_dev(y, "fp32"), want)


def test_in_place_and_deterministic(sb):
    gw, (x, g, b) = workloads.draw_config_groupnorm(3)
    y1, _ = run(sb, gw, x, g, b)
    xd = to_dev(x, gw.dtype)
    y2, _ = run(sb, gw, x, g, b, out=xd, x_dev=xd)
    assert y2.data_ptr() == xd.data_ptr()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("axis", [2, 3])  # patches along H (runs) or W (whole rows per block)
def test_misaligned_input_takes_the_scalar_path(sb, axis):
    gw = _gw((1, 16, 32, 32), "bf16", 4, axis, 4, seed=3)
    x, g, b = workloads.draw_groupnorm(gw)
    xd = to_dev(x, "bf16")
    buf = torch.empty(xd.numel() + 1, dtype=xd.dtype, device=xd.device)
    xs = buf[1:].view(xd.shape)
    xs.copy_(xd)
    y, _ = run(sb, gw, x, g, b, x_dev=xs)
    ref, _, _ = oracle.groupnorm(x, gw.groups, gw.eps, g, b, "bf16")
    ok, rep = compare.groupnorm_check(as_f64(from_dev(y, "bf16"), "bf16"), ref, "bf16")
    assert ok, rep


def test_workspace_too_small_is_rejected(sb):
    x = torch.zeros((1, 8, 16, 16), device="cuda")
    ws = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(sb.SeamBlendError) as ei:
        sb.patch_groupnorm(x, 4, 2, 2, workspace=ws)
    assert ei.value.code == -3


@pytest.mark.parametrize("dtype,offset", [("fp32", 1000.0), ("bf16", 300.0), ("fp16", 200.0)])
def test_large_mean_against_spread(sb, dtype, offset):
    # a mean far above the spread: the shifted sums and the Chan merges must
    # not lose the variance to cancellation
    gw = _gw((2, 16, 24, 40), dtype, 4, 3, 5, seed=21, offset=("fixed", [offset] * 5))
    x, g, b = workloads.draw_groupnorm(gw)
    check(sb, gw, x, g, b, f"offset {offset}")


@pytest.mark.parametrize("G", [1, 48])
def test_one_group_and_one_channel_per_group(sb, G):
    gw = _gw((3, 48, 20, 12), "fp16", G, 2, 3, seed=22)
    x, g, b = workloads.draw_groupnorm(gw)
    check(sb, gw, x, g, b, f"G={G}")


def test_more_planes_than_one_launch_holds(sb):
    # N*C = 131072 (n, c) planes: the normalise pass takes its planes in
    # launches of at most 65535 (the grid's y extent)
    gw = _gw((2, 65536, 4, 4), "bf16", 256, 2, 2, seed=23)
    x, g, b = workloads.draw_groupnorm(gw)
    check(sb, gw, x, g, b, "131072 planes")


@pytest.mark.parametrize("shape,G,axis,P", [
    ((1, 512, 256, 256), 32, 2, 4),   # decoder activation, patches along H
    ((2, 256, 512, 512), 32, 3, 8),   # decoder activation, patches along W (whole-row pass 1)
    ((1, 64, 640, 1024), 2, 2, 3),    # groups of 20,971,520 elements (more than 2^24)
])
def test_fp32_decoder_size_groups(sb, shape, G, axis, P):
    # fp32 at the 1e-5 reading with groups of 10^6 to 2 x 10^7 elements: long
    # per-thread runs and deep merges
    gw = _gw(shape, "fp32", G, axis, P, seed=31)
    x, g, b = workloads.draw_groupnorm(gw)
    check(sb, gw, x, g, b, "fp32 decoder size")


@pytest.mark.parametrize("where", ["first", "first-and-middle"])
@pytest.mark.parametrize("value", [100.0, 1000.0])
def test_fp32_outlying_samples(sb, where, value):
    # N(0,1) groups with an outlier at the group's first element (and its
    # middle one): the statistics must not lose the variance to cancellation
    # against an outlying shift, at the fp32 1e-5 reading
    gw = _gw((1, 32, 32, 256), "fp32", 4, 2, 2, seed=32, offset=None)
    x, g, b = workloads.draw_groupnorm(gw)
    per = x.reshape(gw.shape[0], gw.groups, -1)
    per[:, :, 0] = value
    if where == "first-and-middle":
        per[:, :, per.shape[2] // 2] = value
    check(sb, gw, x, g, b, f"outlier {value} at {where}")


def test_w_split_rows_of_1024_vectors(sb):
    # bf16 rows of 8192 elements split into 4: one row per pass of the
    # 1024-lane statistics block
    gw = _gw((1, 4, 2, 8192), "bf16", 2, 3, 4, seed=24)
    x, g, b = workloads.draw_groupnorm(gw)
    check(sb, gw, x, g, b, "1024-vector rows")


def test_graph_replay_with_changed_inputs(sb):
    # the two passes captured in a HIP graph: every replay, with new x between
    # replays and eager work around them, equals the eager result
    gw, (x, g, b) = workloads.draw_config_groupnorm(4)
    xd, gd, bd = to_dev(x, gw.dtype), to_dev(g, gw.dtype), to_dev(b, gw.dtype)
    plan = sb.PatchGroupNorm(xd, gw.groups, gw.split_axis, gw.n_patches, gw.eps, gd, bd)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        plan()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            plan()
    torch.cuda.synchronize()
    for rep in range(3):
        eager = plan().clone()
        torch.cuda.synchronize()
        plan.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        xd.mul_(-0.5).add_(0.25)  # new input for the next replay
        torch.cuda.synchronize()


def test_concurrent_streams_do_not_interfere(sb):
    # no state is shared between calls: two calls on two streams at once, each
    # with its own workspace, give the serial results
    cases = []
    for cfg in (3, 4):
        gw, (x, g, b) = workloads.draw_config_groupnorm(cfg)
        xd, gd, bd = to_dev(x, gw.dtype), to_dev(g, gw.dtype), to_dev(b, gw.dtype)
        plan = sb.PatchGroupNorm(xd, gw.groups, gw.split_axis, gw.n_patches, gw.eps, gd, bd)
        serial = plan().clone()
        cases.append((plan, serial))
    torch.cuda.synchronize()
    for plan, _ in cases:
        plan.out.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (plan, _), st in zip(cases, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for _ in range(3):
                plan()
    torch.cuda.synchronize()
    for plan, serial in cases:
        assert torch.equal(plan.out.view(torch.int16), serial.view(torch.int16))
