"""Pins of the GroupNorm oracle.

Sources: DistVAE PR "Add tiled VAE parallelism & extended model support" --
the PatchGroupNorm commit (the split norm must equal nn.GroupNorm: global
mean, variance divided by the count; the two bugs were per-rank means and
Bessel's correction), the commit reducing its collectives (squared deviations
about the global mean), and the Patchify commit (first ranks one band longer).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import compare
import oracle
import workloads


def _draw(shape, dtype, seed=0, offset=None, split_axis=2, P=2):
    g = workloads.GroupNormWorkload("t", dtype, shape, 4, split_axis, P, 1e-6, seed,
                                    offset=offset)
    return workloads.draw_groupnorm(g)


def _torch_gn(x, G, eps, gamma, beta, dtype):
    from models import storage_to_f32
    xt = torch.from_numpy(storage_to_f32(x, dtype).astype(np.float64))
    gt = None if gamma is None else torch.from_numpy(storage_to_f32(gamma, dtype).astype(np.float64))
    bt = None if beta is None else torch.from_numpy(storage_to_f32(beta, dtype).astype(np.float64))
    return torch.nn.functional.group_norm(xt, G, gt, bt, eps).numpy()


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 8, 6, 10), (1, 12, 3, 5, 7), (3, 4, 1, 1)])
@pytest.mark.parametrize("affine", [True, False])
def test_groupnorm_equals_torch_float64(dtype, shape, affine):
    x, g, b = _draw(shape, dtype, seed=sum(shape), offset=("uniform", -2, 2))
    if not affine:
        g = b = None
    y, mean, var = oracle.groupnorm(x, 4, 1e-6, g, b, dtype)
    ref = _torch_gn(x, 4, 1e-6, g, b, dtype)
    assert np.max(np.abs(y - ref)) <= 1e-12


def test_config1_groupnorm_equals_torch_float64():
    gw, (x, g, b) = workloads.draw_config_groupnorm(1)
    y, _, _ = oracle.groupnorm(x, gw.groups, gw.eps, g, b, gw.dtype)
    ref = _torch_gn(x, gw.groups, gw.eps, g, b, gw.dtype)
    assert np.max(np.abs(y - ref)) <= 1e-12


@pytest.mark.parametrize("split_axis,P", [(2, 3), (3, 4), (2, 7), (3, 1), (2, 11)])
def test_patch_stats_match_numpy_per_patch(split_axis, P):
    x, _, _ = _draw((2, 8, 9, 10), "fp32", seed=P, offset=("uniform", -2, 2), split_axis=split_axis, P=P)
    st = oracle.patch_stats(x, 4, split_axis, P, "fp32")
    xr = x.astype(np.float64).reshape(2, 4, 2, 9, 10)
    parts = np.array_split(np.arange(x.shape[split_axis]), P)
    for p, idx in enumerate(parts):
        sl = np.take(xr, idx, axis=split_axis + 1)
        cnt = sl[0, 0].size
        assert np.all(st[:, :, p, 0] == cnt)
        if cnt:
            m = sl.reshape(2, 4, -1).mean(axis=2)
            m2 = ((sl.reshape(2, 4, -1) - m[..., None]) ** 2).sum(axis=2)
            assert np.allclose(st[:, :, p, 1], m, rtol=0, atol=1e-13)
            assert np.allclose(st[:, :, p, 2], m2, rtol=1e-12, atol=1e-12)
        else:
            assert np.all(st[:, :, p, 1:] == 0)


def test_patch_split_is_array_split():
    for L in range(0, 40):
        for P in range(1, 9):
            bounds = workloads.patch_bounds(L, P)
            sizes = [e - s for s, e in bounds]
            assert sizes == [len(a) for a in np.array_split(np.arange(L), P)]


@pytest.mark.parametrize("shape,split_axis,P", [((2, 8, 16, 6), 2, 2), ((1, 8, 5, 7, 9), 3, 4),
                                                  ((1, 8, 5, 7, 9), 4, 3), ((1, 8, 5, 7, 9), 2, 8)])
def test_chan_merge_equals_direct_statistics(shape, split_axis, P):
    x, _, _ = _draw(shape, "fp32", seed=3, offset=("uniform", -2, 2), split_axis=split_axis,
                    P=min(P, shape[split_axis]))
    st = oracle.patch_stats(x, 4, split_axis, P, "fp32")
    merged = oracle.chan_merge(st)
    _, mean, var = oracle.groupnorm(x, 4, 1e-6, None, None, "fp32")
    n = merged[..., 0]
    assert np.all(n == x[0].size // 4)
    assert np.allclose(merged[..., 1], mean, rtol=0, atol=1e-13)
    assert np.allclose(merged[..., 2] / n, var, rtol=1e-12, atol=0)


def test_two_equal_patches_textbook_identity():
    # sigma^2 = (v1 + v2)/2 + (m1 - m2)^2 / 4 for two patches of equal size
    gw, (x, g, b) = workloads.draw_config_groupnorm(1)
    st = oracle.patch_stats(x, gw.groups, gw.split_axis, gw.n_patches, gw.dtype)
    _, mean, var = oracle.groupnorm(x, gw.groups, gw.eps, g, b, gw.dtype)
    v1, v2 = st[..., 0, 2] / st[..., 0, 0], st[..., 1, 2] / st[..., 1, 0]
    m1, m2 = st[..., 0, 1], st[..., 1, 1]
    assert np.allclose(var, (v1 + v2) / 2 + (m1 - m2) ** 2 / 4, rtol=1e-12, atol=0)
    # the +3.0 offset of the second patch makes the between-patch term ~2.25
    assert np.all(np.abs((m1 - m2) ** 2 / 4 - 2.25) < 0.3)


def test_constant_group_gives_beta_exactly():
    x = np.full((1, 8, 4, 4), 1.75, np.float32)
    g = np.linspace(0.5, 1.5, 8).astype(np.float32)
    b = np.linspace(-1, 1, 8).astype(np.float32)
    y, mean, var = oracle.groupnorm(x, 4, 1e-6, g, b, "fp32")
    assert np.all(var == 0) and np.all(mean == 1.75)
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64)[None, :, None, None], y.shape))


def test_single_patch_is_plain_groupnorm():
    x, _, _ = _draw((2, 8, 6, 6), "bf16", seed=9)
    st = oracle.patch_stats(x, 4, 2, 1, "bf16")
    _, mean, var = oracle.groupnorm(x, 4, 1e-6, None, None, "bf16")
    assert np.allclose(st[..., 0, 1], mean, atol=1e-13, rtol=0)
    assert np.allclose(st[..., 0, 2] / st[..., 0, 0], var, rtol=1e-12)


# ---------------------------------------------------------------------------
# planted mistakes (on the CPU, in the oracle's arithmetic): the comparator
# used by the GPU parity tests must reject both historical bugs
# ---------------------------------------------------------------------------
def _normalise(x, mean, var, eps, gamma, beta, G, dtype):
    from models import storage_to_f32
    xv = storage_to_f32(x, dtype).astype(np.float64)
    N, C = xv.shape[:2]
    xg = xv.reshape(N, G, -1)
    y = (xg - mean[..., None]) / np.sqrt(var[..., None] + eps)
    y = y.reshape(xv.shape)
    gm = storage_to_f32(gamma, dtype).astype(np.float64)
    bt = storage_to_f32(beta, dtype).astype(np.float64)
    shp = (1, C) + (1,) * (xv.ndim - 2)
    return y * gm.reshape(shp) + bt.reshape(shp)


@pytest.mark.parametrize("cfg", [1, 3])
def test_comparator_rejects_per_patch_mean_and_bessel(cfg):
    gw, (x, g, b) = workloads.draw_config_groupnorm(cfg)
    if cfg == 3:  # a slice of config 3 keeps this fast
        x = np.ascontiguousarray(x[:, :64])
        g, b = g[:64], b[:64]
        gw = workloads.GroupNormWorkload(gw.name, gw.dtype, x.shape, 4, gw.split_axis,
                                         gw.n_patches, gw.eps, gw.seed)
    y, mean, var = oracle.groupnorm(x, gw.groups, gw.eps, g, b, gw.dtype)
    st = oracle.patch_stats(x, gw.groups, gw.split_axis, gw.n_patches, gw.dtype)
    n = st[..., 0].sum(axis=-1)
    ok, _ = compare.groupnorm_check(y, y, gw.dtype)
    assert ok
    # bug 1: variance about each patch's own mean (between-patch term dropped)
    var_pp = st[..., 2].sum(axis=-1) / n
    y1 = _normalise(x, mean, var_pp, gw.eps, g, b, gw.groups, gw.dtype)
    assert not compare.groupnorm_check(y1, y, gw.dtype)[0]
    # bug 2: Bessel's correction (divide by n - 1)
    var_b = var * n / (n - 1)
    y2 = _normalise(x, mean, var_b, gw.eps, g, b, gw.groups, gw.dtype)
    if gw.dtype == "fp32":
        assert not compare.groupnorm_check(y2, y, gw.dtype)[0]
    # sanity: the comparator accepts the oracle's own normalisation rebuilt here
    y0 = _normalise(x, mean, var, gw.eps, g, b, gw.groups, gw.dtype)
    assert compare.groupnorm_check(y0, y, gw.dtype)[0]
