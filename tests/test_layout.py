"""Tile layouts along one axis: the oracle against the layouts and properties
the pages state, and the library's planner against the oracle (host code, so
these run without a GPU)."""
from __future__ import annotations

import json
import os
import random

import pytest

from oracle import layout as ol

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "layout_pages.json")
PAGES = json.load(open(GOLDEN))


@pytest.fixture(scope="module")
def sb():
    import seam_blending_patch_amd as m
    return m


def lib_tiles(sb, L, rule, params):
    o, e = sb.vae_tile_layout(L, rule, params)
    return list(zip(o, e))


@pytest.mark.parametrize("case", PAGES["layouts"], ids=lambda c: f"{c['rule']}-{c['L']}")
def test_oracle_reproduces_the_pages_layouts(case):
    tiles = ol.layout(case["L"], case["rule"], case["params"])
    assert [e for _, e in tiles] == case["extents"], case["cite"]
    if "origins" in case:
        assert [o for o, _ in tiles] == case["origins"], case["cite"]
    if "decoded" in case:
        assert ol.decoded(tiles) == case["decoded"]
    if "calls_2d" in case:
        assert len(tiles) ** 2 == case["calls_2d"]
    assert ol.covers(case["L"], tiles, 0)


@pytest.mark.parametrize("case", PAGES["decoded_ratio"], ids=lambda c: c["rule"])
def test_oracle_decoded_area_against_the_pages(case):
    tiles = ol.layout(case["L"], case["rule"], case["params"])
    ratio = (ol.decoded(tiles) / case["L"]) ** 2
    assert abs(ratio - case["ratio_2d"]) <= case["tol"], (ratio, case["cite"])


def test_oracle_smallest_side_picks_the_printed_tile_sides():
    fp = PAGES["smallest_side_fixed_points"]
    for c in fp["cases"]:
        for s in c["sides"]:
            tiles = ol.smallest_side(c["L"], fp["overlap"], s)
            assert {e for _, e in tiles} == {min(s, c["L"])}, (c, s)
            # and one tile fewer of that side cannot cover
            n = len(tiles)
            if n > 1:
                assert not any(ol.covers(c["L"], ol.spread(c["L"], t, n - 1), fp["overlap"])
                               for t in range(1, s + 1))


def _sliver_lengths():
    return [L for L in range(129, 420) if ol.stock(L, 128, 96)[-1][1] < 32]


@pytest.mark.parametrize("M", [128, 192, 256])
def test_oracle_sliver_rule_has_the_properties_the_pages_test(M):
    # section Tests: at every sliver length from 129 to 419 latents and three
    # budgets, fewer decoder calls than stock, no more decoded latents per
    # side up to rounding (under one latent per tile), and every overlap at
    # least 32
    lengths = _sliver_lengths()
    assert len(lengths) > 50
    for L in lengths:
        st = ol.stock(L, 128, 96)
        fc = ol.fewest_calls(L, 128, 96, 32, M)
        assert len(fc) < len(st), L
        assert ol.decoded(fc) <= ol.decoded(st) + len(fc) - 1, L  # up to rounding
        assert all(x >= 32 for x in ol.overlaps(fc)), L
        assert ol.covers(L, fc, 32)
        assert max(e for _, e in fc) <= M


def test_oracle_edge_aligned_is_full_and_ends_at_the_edge():
    # commit bringing seam-free tiles to Qwen-Image-2.1: every tile full size,
    # the last ending at the edge, overlaps at least 16, the fewest such tiles
    for L in range(1, 400):
        tiles = ol.edge_aligned(L, 32, 16)
        if L <= 32:
            assert tiles == [(0, L)]
            continue
        assert all(e == 32 for _, e in tiles)
        assert tiles[-1][0] + 32 == L
        assert min(ol.overlaps(tiles)) >= 16
        # fewest: n - 1 tiles of 32 cannot reach L with that overlap
        n = len(tiles)
        assert (n - 1) * 32 - (n - 2) * 16 < L
        # the gaps differ by at most one latent
        gaps = [b[0] - a[0] for a, b in zip(tiles, tiles[1:])]
        assert max(gaps) - min(gaps) <= 1


def test_oracle_checker_rejects_gaps_repeats_and_short_tiles():
    bad = [(0, 32), (33, 32)]
    assert not ol.covers(65, bad, 0)
    assert not ol.covers(64, [(0, 32), (16, 32), (32, 31)], 16)
    assert not ol.covers(64, [(0, 32), (0, 32), (32, 32)], 16)


# ---------------------------------------------------------------- library

PARAMS = {
    "stock": [[16, 12], [128, 96], [64, 48], [12, 9], [7, 7], [1, 1], [33, 5]],
    "edge_aligned": [[32, 16], [64, 32], [128, 32], [5, 0], [9, 8], [1, 0]],
    "fewest_calls": [[128, 96, 32, 128], [128, 96, 32, 192], [128, 96, 32, 256], [64, 48, 16, 64],
                     [16, 12, 4, 40], [32, 24, 8, 33]],
    "smallest_side": [[32, 128], [16, 32], [16, 44], [16, 72], [0, 10], [8, 9], [4, 500]],
    "auto": [[128, 96, 32, 16], [16, 12, 32, 16], [12, 9, 32, 16], [64, 48, 32, 16], [32, 16, 32, 16]],
}


@pytest.mark.parametrize("rule", sorted(PARAMS))
def test_library_matches_oracle_at_every_length(sb, rule):
    for p in PARAMS[rule]:
        for L in range(1, 450):
            try:
                want = ol.layout(L, rule, p)
            except ValueError:
                with pytest.raises(sb.SeamBlendError):
                    sb.vae_tile_layout(L, rule, p)
                continue
            assert lib_tiles(sb, L, rule, p) == want, (rule, p, L)


def test_library_matches_oracle_on_random_parameters(sb):
    rng = random.Random(7)
    # sides at least 8 latents above the overlap keep the oracle's search short
    for _ in range(400):
        rule = rng.choice(sorted(PARAMS))
        L = rng.randint(1, 1200)
        T = rng.randint(1, 300)
        S = rng.randint(1, T)
        ov = rng.randint(0, max(0, T - 8))
        M = rng.randint(ov + 8, ov + 300)
        p = {"stock": [T, S], "edge_aligned": [T, ov], "fewest_calls": [T, S, ov, M],
             "smallest_side": [ov, M], "auto": [T, S, rng.randint(1, 64), rng.randint(0, 32)]}[rule]
        try:
            want = ol.layout(L, rule, p)
        except ValueError:
            with pytest.raises(sb.SeamBlendError):
                sb.vae_tile_layout(L, rule, p)
            continue
        assert lib_tiles(sb, L, rule, p) == want, (rule, p, L)


@pytest.mark.parametrize("rule,params", [
    ("stock", [0, 1]), ("stock", [4, 0]), ("stock", [4, 5]),
    ("edge_aligned", [8, 8]), ("edge_aligned", [8, -1]),
    ("fewest_calls", [0, 1, 0, 8]), ("smallest_side", [8, 8]), ("auto", [16, 12, 0, 0]),
])
def test_library_rejects_bad_parameters(sb, rule, params):
    with pytest.raises(sb.SeamBlendError) as ei:
        sb.vae_tile_layout(100, rule, params)
    assert ei.value.code == -1


def test_single_tile_canvas_ignores_the_overlap(sb):
    # a canvas no wider than the tile is one tile, whatever overlap is asked
    # for (a lone tile has no neighbour); with several tiles an overlap that
    # reaches the tile side is a bad parameter
    for L, rule, p in [(8, "edge_aligned", [8, 8]), (5, "edge_aligned", [8, 20]),
                       (2, "auto", [1, 1, 2, 2]), (64, "auto", [16, 16, 64, 64])]:
        assert ol.layout(L, rule, p) == [(0, L)], (L, rule, p)
        assert lib_tiles(sb, L, rule, p) == [(0, L)], (L, rule, p)
    for L, rule, p in [(9, "edge_aligned", [8, 8]), (65, "auto", [16, 16, 64, 64])]:
        with pytest.raises(sb.SeamBlendError) as ei:
            sb.vae_tile_layout(L, rule, p)
        assert ei.value.code == -1


def test_library_rejects_a_layout_beyond_capacity(sb):
    with pytest.raises(sb.SeamBlendError) as ei:
        sb.vae_tile_layout(1000, "stock", [2, 1], max_tiles=16)
    assert ei.value.code == -1


def test_extreme_parameters_fail_fast(sb):
    # canvas and parameters beyond 2^30, and layouts with far more tiles than
    # the output arrays hold, are rejected without walking the tiles
    import time
    t0 = time.perf_counter()
    for rule, L, p in [("fewest_calls", 1 << 30, [1 << 30, 1, 0, 5]),
                       ("auto", 1 << 30, [1 << 20, 1, 1, 0]),
                       ("stock", 1 << 30, [2, 1]),
                       ("edge_aligned", 1 << 30, [2, 1]),
                       ("smallest_side", 1 << 30, [1, 2]),
                       ("stock", (1 << 30) + 1, [16, 12]),
                       ("fewest_calls", 100, [128, 96, 1 << 31, 128]),
                       ("auto", 100, [16, 12, -1, 0])]:
        with pytest.raises(sb.SeamBlendError):
            sb.vae_tile_layout(L, rule, p, max_tiles=64)
    assert time.perf_counter() - t0 < 1.0
