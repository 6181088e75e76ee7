"""Pins of the normalised-ramp oracle (oracle.ramp_blend / oracle.ramp_weight)
against what the pages and arithmetic fix, independent of the oracle's code:
hand-computed weights of the stated margin and ramp, tiles that agree,
single-tile regions, the zero-weight band, mirror symmetry, weights that sum
to 1 on the pages' layouts at every length and ratio, and a factored
per-axis normalisation computed a different way."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import layout as ol
import workloads as W

# unsloth Studio PR "size seam-free VAE tiles from measured peaks", the
# Qwen-Image-2.1 wide-tile commit: no weight within 4 latents of a shared
# edge, full weight after the next 8
M, R = 4, 8



def test_hand_computed_weights_of_two_overlapping_tiles():
    # tiles [0, 32) and [16, 48) along W, one row; ratio 1.
    # at x = 24: tile 0 is 7 from its shared upper edge -> (7 - 4) / 8 = 3/8,
    # tile 1 is 8 from its shared lower edge -> (8 - 4) / 8 = 1/2;
    # normalised 3/7 and 4/7.
    assert oracle.ramp_weight(24, 0, 32, 0, 2, M, R) == 0.375
    assert oracle.ramp_weight(24, 16, 32, 1, 2, M, R) == 0.5
    a, b = 1.0, 8.0
    tiles = [np.full((1, 1, 1, 32), a, np.float32), np.full((1, 1, 1, 32), b, np.float32)]
    out = oracle.ramp_blend(tiles, (1, 1), [0], [1], [0, 16], [32, 32], (M, M), (R, R), "fp32")
    assert abs(out[0, 0, 0, 24] - (3 * a + 4 * b) / 7) < 1e-14
    # within 4 of tile 1's lower edge (x <= 20) only tile 0 has weight
    for x in range(16, 21):
        assert out[0, 0, 0, x] == a
    # within 4 of tile 0's upper edge (x >= 27) only tile 1 has weight
    for x in range(27, 32):
        assert out[0, 0, 0, x] == b
    # the canvas edges are not shared: full weight up to them
    assert oracle.ramp_weight(0, 0, 32, 0, 2, M, R) == 1.0
    assert oracle.ramp_weight(47, 16, 32, 1, 2, M, R) == 1.0
    # the ramp is linear: one position further from the edge adds 1/8
    for d in range(M, M + R + 1):
        assert oracle.ramp_weight(16 + d, 16, 32, 1, 2, M, R) == (d - M) / R


def test_tiles_cut_from_one_image_reproduce_it():
    rng = np.random.default_rng(5)
    for ratio, L, layout in [(16, 64, (32, 16)), (8, 50, (32, 16)), (1, 128, (64, 32))]:
        tiles_o = [o for o, _ in ol.edge_aligned(L, *layout)]
        t = layout[0]
        img = rng.normal(size=(2, 3, L * ratio, L * ratio)).astype(np.float32)
        o_px = [o * ratio for o in tiles_o]
        tiles = [np.ascontiguousarray(img[:, :, a:a + t * ratio, b:b + t * ratio])
                 for a in o_px for b in o_px]
        out = oracle.ramp_blend(tiles, (2, 3), o_px, [t * ratio] * len(o_px), o_px,
                                [t * ratio] * len(o_px), (M * ratio,) * 2, (R * ratio,) * 2, "fp32")
        assert np.max(np.abs(out - img)) <= 4e-16 * np.max(np.abs(img)) * 8


def test_single_tile_regions_copy_and_constant_stays_constant():
    w = W.RAMP_WORKLOADS["flux-1600-bf16"]
    small = W.RampWorkload("t", "fp32", (1, 2), [0, 40], [60, 60], [0, 40], [60, 60],
                           (2, 2), (4, 4), seed=3, clamp=None)
    tiles = W.draw_ramp_tiles(small)
    out = oracle.ramp_blend(tiles, small.lead, small.origins_h, small.extents_h, small.origins_w,
                            small.extents_w, small.margin, small.ramp, "fp32")
    # rows/cols < 40 + 2 + 1 only tile row/col 0 has weight; >= 60 - 2 - 1 only the second
    np.testing.assert_array_equal(out[..., :43, :43], tiles[0][..., :43, :43].astype(np.float64))
    np.testing.assert_array_equal(out[..., 57:, 57:], tiles[3][..., 17:, 17:].astype(np.float64))
    const = [np.full(t.shape, 0.625, np.float32) for t in tiles]
    out = oracle.ramp_blend(const, small.lead, small.origins_h, small.extents_h, small.origins_w,
                            small.extents_w, small.margin, small.ramp, "fp32")
    assert np.max(np.abs(out - 0.625)) < 1e-15
    assert w.out_shape == (1, 3, 1600, 1600)


def test_values_in_the_zero_weight_band_do_not_matter():
    small = W.RampWorkload("t", "fp32", (1, 1), [0, 20], [36, 36], [0, 24], [40, 40],
                           (3, 3), (5, 5), seed=4, clamp=None)
    tiles = W.draw_ramp_tiles(small)
    args = (small.lead, small.origins_h, small.extents_h, small.origins_w, small.extents_w,
            small.margin, small.ramp, "fp32")
    ref = oracle.ramp_blend(tiles, *args)
    poked = [t.copy() for t in tiles]
    # tile (1, 1): rows and columns within 3 of its shared lower edges weigh 0
    poked[3][..., :4, :] = 1e6
    poked[3][..., :, :4] = -1e6
    # tile (0, 0): within 3 of its shared upper edges
    poked[0][..., -4:, :] = 7e5
    np.testing.assert_array_equal(oracle.ramp_blend(poked, *args), ref)
    # one position further in does matter
    poked[3][..., 4, 10] = 1e6
    assert not np.array_equal(oracle.ramp_blend(poked, *args), ref)


def test_mirror_symmetry():
    # flipping the canvas turns each tile's lower shared edge into the
    # mirrored tile's upper one: the blend of the flipped tiles is the flipped
    # blend (an off-by-one in either edge distance breaks this)
    small = W.RampWorkload("t", "fp32", (1, 2), [0, 9, 21], [30, 30, 30], [0, 13], [33, 33],
                           (2, 1), (6, 3), seed=8, clamp=None)
    rng = np.random.default_rng(8)
    tiles = [rng.normal(size=small.tile_shape(i, j)).astype(np.float32)
             for i in range(3) for j in range(2)]
    ref = oracle.ramp_blend(tiles, small.lead, small.origins_h, small.extents_h, small.origins_w,
                            small.extents_w, small.margin, small.ramp, "fp32")
    LH, LW = ref.shape[-2:]
    fo_h = [LH - o - e for o, e in zip(small.origins_h, small.extents_h)][::-1]
    fo_w = [LW - o - e for o, e in zip(small.origins_w, small.extents_w)][::-1]
    ftiles = [np.ascontiguousarray(tiles[i * 2 + j][..., ::-1, ::-1])
              for i in (2, 1, 0) for j in (1, 0)]
    got = oracle.ramp_blend(ftiles, small.lead, fo_h, small.extents_h[::-1], fo_w,
                            small.extents_w[::-1], small.margin, small.ramp, "fp32")
    assert np.max(np.abs(got[..., ::-1, ::-1] - ref)) < 1e-14


@pytest.mark.parametrize("ratio", [8, 16, 32])
def test_weights_sum_to_one_on_the_floor_layout_at_every_length(ratio):
    # section Tests: wide tiles full and edge-aligned, weights summing to 1, at
    # every length and ratio; every position has a tile with weight
    for L in range(33, 200):
        tiles = ol.edge_aligned(L, 32, 16)
        o = [a * ratio for a, _ in tiles]
        s = [e * ratio for _, e in tiles]
        n = len(o)
        for p in range(0, L * ratio, max(1, ratio // 2)):
            w = [oracle.ramp_weight(p, o[k], s[k], k, n, M * ratio, R * ratio) for k in range(n)]
            tot = sum(w)
            assert tot > 0, (L, ratio, p)
            assert abs(sum(x / tot for x in w) - 1.0) < 1e-15


def test_matches_a_factored_per_axis_normalisation():
    # the 2-D weight is a product of axis weights, so its normalisation factors;
    # compute it that way with numpy and compare
    w = W.random_ramp_workload(11, "fp32", lead=(2, 2), max_tiles=4, max_ext=40)
    tiles = W.draw_ramp_tiles(w)
    ref = oracle.ramp_blend(tiles, w.lead, w.origins_h, w.extents_h, w.origins_w, w.extents_w,
                            w.margin, w.ramp, "fp32")
    LH, LW = ref.shape[-2:]

    def axis_table(origins, extents, m, r, L):
        n = len(origins)
        t = np.zeros((n, L))
        for k, (o, s) in enumerate(zip(origins, extents)):
            p = np.arange(o, o + s)
            f = np.ones(s)
            if k > 0:
                f *= np.clip((p - o - m) / r, 0, 1)
            if k < n - 1:
                f *= np.clip((o + s - 1 - p - m) / r, 0, 1)
            t[k, o:o + s] = f
        return t / t.sum(axis=0, keepdims=True)

    th = axis_table(w.origins_h, w.extents_h, w.margin[0], w.ramp[0], LH)
    tw = axis_table(w.origins_w, w.extents_w, w.margin[1], w.ramp[1], LW)
    acc = np.zeros(ref.shape)
    nw = len(w.origins_w)
    for i, (oh, sh) in enumerate(zip(w.origins_h, w.extents_h)):
        for j, (ow, sw) in enumerate(zip(w.origins_w, w.extents_w)):
            acc[..., oh:oh + sh, ow:ow + sw] += (th[i, oh:oh + sh, None] * tw[j, None, ow:ow + sw]
                                                 * tiles[i * nw + j].astype(np.float64))
    assert np.max(np.abs(acc - ref)) < 1e-12


def test_rejects_an_uncovered_position():
    # margin 4: tile 0 weighs 0 where its distance to the shared edge is <= 4,
    # tile 1 likewise; an overlap of 9 leaves its middle position to neither
    tiles = [np.ones((1, 1, 1, 20), np.float32), np.ones((1, 1, 1, 20), np.float32)]
    with pytest.raises(ValueError):
        oracle.ramp_blend(tiles, (1, 1), [0], [1], [0, 11], [20, 20], (4, 4), (8, 8), "fp32")
    # an overlap of 10 leaves every position covered
    oracle.ramp_blend(tiles, (1, 1), [0], [1], [0, 10], [20, 20], (4, 4), (8, 8), "fp32")
