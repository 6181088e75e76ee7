"""Pins of the blend + stitch oracle against things other than itself.

Each test names what fixes the expected value: an IEEE/library conversion, an
exact rational computation, an invariant of the crossfade, a special case that
reduces to slicing and concatenation, or agreement with two independent
brute-force models (literal torch, per-element closed form).  Sources: diffusers
issue "[Proposal] Vectorize tiled VAE blending while preserving rounding and
CUDA graph replay", section "Proposed scope" (clamping, in-place output,
per-product rounding, float64 coefficients).
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction

import numpy as np
import pytest
import torch

import compare
import models
import oracle
import workloads


# ---------------------------------------------------------------------------
# storage conversions: library routines fix the answer
# ---------------------------------------------------------------------------
def _f32_samples(n=400_000, seed=0):
    rng = np.random.default_rng(seed)
    raw = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    v = raw.view(np.float32)
    v = v[np.isfinite(v)]
    # exact binary16 midpoints (ties), and values around the f16 subnormal range
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = h[:-1].view(np.float16).astype(np.float64)
    hi = h[1:].view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    small = (rng.uniform(-1, 1, 100_000) * 2.0 ** rng.integers(-30, -10, 100_000)).astype(np.float32)
    big = (rng.uniform(-1, 1, 50_000) * 70000).astype(np.float32)
    return np.concatenate([v, mids, -mids, small, big])


def test_f16_rounding_matches_numpy():
    v = _f32_samples()
    got = oracle.round_to_storage_bits(v, "fp16")
    with np.errstate(over="ignore"):  # values beyond binary16 range round to infinity on purpose
        want = v.astype(np.float16).view(np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_rounding_matches_torch():
    v = _f32_samples()
    got = oracle.round_to_storage_bits(v, "bf16")
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # exact bf16 ties too
    b = np.arange(0, 0x7F80, dtype=np.uint32)
    mids = ((b << 16) | 0x8000).view(np.float32)
    got2 = oracle.round_to_storage_bits(mids, "bf16")
    want2 = torch.from_numpy(mids).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(got2, want2)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_widening_is_exact_for_every_pattern(dtype):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen_storage_bits(pats, dtype)
    if dtype == "fp16":
        want = pats.view(np.float16).astype(np.float32)
    else:
        want = (pats.astype(np.uint32) << 16).view(np.float32)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(want))


# ---------------------------------------------------------------------------
# coefficients: correctly rounded k/e and (e-k)/e, never 1 - w_b in fp32
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("e", [1, 2, 3, 5, 7, 12, 16, 64, 100, 127, 128, 333, 1000])
def test_coefficients_are_correctly_rounded_rationals(e):
    wa, wb = oracle.coefficients(e)
    for k in range(e):
        assert wb[k] == models.correctly_rounded_f32(Fraction(k, e)), (e, k)
        assert wa[k] == models.correctly_rounded_f32(Fraction(e - k, e)), (e, k)


def test_wa_is_not_one_minus_wb_in_fp32():
    # rounding 1 - k/e once from double differs from 1 - fp32(k/e) in fp32
    diffs = 0
    for e in range(2, 200):
        wa, wb = oracle.coefficients(e)
        diffs += int(np.sum(wa != (np.float32(1.0) - wb)))
    assert diffs > 0
    wa, wb = oracle.coefficients(3)
    assert wa[1] == np.float32(2.0 / 3.0)
    assert wa[1] != np.float32(1.0) - np.float32(1.0 / 3.0)


def test_power_of_two_extent_coefficients_are_exact_dyadics():
    wa, wb = oracle.coefficients(16)
    assert np.array_equal(wb, np.arange(16, dtype=np.float32) / 16)
    assert np.array_equal(wa, (16 - np.arange(16, dtype=np.float32)) / 16)


# ---------------------------------------------------------------------------
# single crossfade: endpoints, exact dyadic cases, per-product rounding
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_endpoint_w0_returns_a(dtype):
    rng = np.random.default_rng(5)
    vals = models.rn(rng.normal(0, 0.5, 2000).astype(np.float32), dtype)
    for a, b in zip(vals[:1000], vals[1000:]):
        out = oracle.crossfade(float(a), float(b), 1.0, 0.0, dtype)
        assert np.float32(out) == a
    # sign of zero: a = -0, b >= 0 gives +0; a = -0, b < 0 gives -0
    assert np.signbit(oracle.crossfade(-0.0, 0.25, 1.0, 0.0, dtype)) == False  # noqa: E712
    assert np.signbit(oracle.crossfade(-0.0, -0.25, 1.0, 0.0, dtype)) == True  # noqa: E712


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_endpoint_last_row_exact_for_dyadics(dtype):
    # e = 16, k = 15: w_a = 1/16, w_b = 15/16; short dyadic inputs make every
    # step exact, so out = a/16 + 15 b/16 exactly
    wa, wb = oracle.coefficients(16)
    for a, b in [(1.0, -0.5), (0.75, 0.25), (-1.0, 1.0), (0.5, 0.5), (-0.125, 0.875)]:
        exact = Fraction(a) / 16 + Fraction(b) * 15 / 16
        assert Fraction(oracle.crossfade(a, b, float(wa[15]), float(wb[15]), dtype)) == exact


def test_per_product_rounding_is_visible_in_fp16():
    # a*w_a and b*w_b are each rounded to fp16 before the sum; rounding only
    # the sum would give a different fp16 here.  Expected values by exact
    # rational arithmetic with one correct rounding at each stated place.
    e, k = 3, 1
    wa, wb = oracle.coefficients(e)
    found = 0
    rng = np.random.default_rng(11)
    for _ in range(4000):
        a, b = (float(np.float16(v)) for v in rng.normal(0, 0.5, 2))
        fa, fb = Fraction(float(wa[k])), Fraction(float(wb[k]))

        def rn16(x):
            return Fraction(float(np.float16(models.correctly_rounded_f32(x))))

        pa = rn16(Fraction(a) * fa)
        pb = rn16(Fraction(b) * fb)
        want = rn16(pa + pb)
        got = Fraction(oracle.crossfade(a, b, float(wa[k]), float(wb[k]), "fp16"))
        assert got == want
        once = rn16(models.correctly_rounded_f32(Fraction(a) * fa) + models.correctly_rounded_f32(Fraction(b) * fb))
        found += int(once != want)
    assert found > 0  # the two roundings do differ on some inputs


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_crossfade_within_rounding_bound_of_exact(dtype):
    # |out - (a(1-k/e) + b k/e)| is bounded by the roundings (coefficients,
    # two products, the sum); a dropped term or swapped weight breaks it
    rng = np.random.default_rng(3)
    for e in (5, 16, 128):
        wa, wb = oracle.coefficients(e)
        for _ in range(300):
            k = int(rng.integers(0, e))
            a, b = (float(v) for v in models.rn(rng.normal(0, 0.5, 2).astype(np.float32), dtype))
            exact = Fraction(a) * Fraction(e - k, e) + Fraction(b) * Fraction(k, e)
            got = Fraction(oracle.crossfade(a, b, float(wa[k]), float(wb[k]), dtype))
            m = max(abs(a), abs(b), 2.0 ** -14)
            bound = Fraction(2 * float(compare.ulp(np.array([m]), dtype)[0]))
            assert abs(got - exact) <= bound, (dtype, e, k, a, b)


# ---------------------------------------------------------------------------
# whole-grid invariants and special cases
# ---------------------------------------------------------------------------
def _wl(dtype, ext_h, ext_w, E, R, ndim=4, ext_t=(1,), Et=0, Rt=1, N=1, C=2, seed=0):
    return workloads.BlendWorkload("t", dtype, ndim, N, C, list(ext_t), list(ext_h), list(ext_w),
                                   (Et, E, E), (Rt, R, R), seed=seed)


def _slice_tiles_from_image(w, img):
    """Tiles cut from one image at their origins: neighbours agree in overlaps."""
    tiles = []
    nt, nh, nw = w.grid
    for tau in range(nt):
        for i in range(nh):
            for j in range(nw):
                f0, y0, x0 = tau * w.row_limit[0], i * w.row_limit[1], j * w.row_limit[2]
                t = img[:, :, f0:f0 + w.ext_t[tau], y0:y0 + w.ext_h[i], x0:x0 + w.ext_w[j]]
                if w.ndim == 4:
                    t = t[:, :, 0]
                tiles.append(np.ascontiguousarray(t))
    return tiles


@pytest.mark.parametrize("dtype,scale", [("fp32", 64), ("fp16", 64), ("bf16", 8)])
@pytest.mark.parametrize("ndim", [4, 5])
def test_agreeing_tiles_reproduce_image_exactly_for_dyadics(dtype, scale, ndim):
    # e a power of two and values k/scale with few bits: every product and sum
    # is exact, so tiles cut from one image blend back into that image
    if ndim == 4:
        w = _wl(dtype, [48, 48, 20], [48, 48, 48, 30], 16, 32)
    else:
        w = _wl(dtype, [48, 30], [48, 48, 30], 16, 32, ndim=5, ext_t=(12, 12, 5), Et=4, Rt=8)
    LT, LH, LW = oracle.output_extents(w.ext_t, w.ext_h, w.ext_w, w.row_limit)
    rng = np.random.default_rng(1)
    img = rng.integers(-scale, scale + 1, size=(w.N, w.C, LT, LH, LW)) / scale
    img_s = models.f32_to_storage(img.astype(np.float32), dtype)
    out = oracle.blend_workload(w, _slice_tiles_from_image(w, img_s))
    want = img_s if ndim == 5 else img_s[:, :, 0]
    compare.assert_bitexact(out, want, dtype, "agree-identity")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_agreeing_tiles_within_one_ulp_in_general(dtype):
    w = _wl(dtype, [40, 40, 40], [40, 40, 17], 13, 27)
    LT, LH, LW = oracle.output_extents(w.ext_t, w.ext_h, w.ext_w, w.row_limit)
    rng = np.random.default_rng(2)
    img = models.f32_to_storage(rng.normal(0, 0.5, (1, 2, LT, LH, LW)).astype(np.float32), dtype)
    out = models.storage_to_f32(oracle.blend_workload(w, _slice_tiles_from_image(w, img)), dtype)
    ref = models.storage_to_f32(img[:, :, 0], dtype)
    d = np.abs(out.astype(np.float64) - ref)
    assert np.all(d <= compare.ulp(ref, dtype) * (2 if dtype == "fp32" else 1))
    assert np.any(d > 0)  # not bit-exact in general: that is expected


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_constant_image_stays_constant(dtype):
    w = _wl(dtype, [40, 40, 11], [40, 40], 16, 24)
    tiles = [np.full(w.tile_shape(0, i, j), 0.375, dtype=np.float32) for i in range(3) for j in range(2)]
    tiles = [models.f32_to_storage(t, dtype) for t in tiles]
    out = models.storage_to_f32(oracle.blend_workload(w, tiles), dtype)
    assert np.all(out == np.float32(0.375))
    # a non-dyadic constant stays within one step
    c = float(models.rn(np.array([0.3], np.float32), dtype)[0])
    tiles = [models.f32_to_storage(np.full(w.tile_shape(0, i, j), c, np.float32), dtype)
             for i in range(3) for j in range(2)]
    out = models.storage_to_f32(oracle.blend_workload(w, tiles), dtype)
    assert np.all(np.abs(out - c) <= compare.ulp(np.array([c]), dtype)[0] * (2 if dtype == "fp32" else 1))


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_single_tile_is_a_copy(dtype):
    w = _wl(dtype, [37], [29], 8, 20, N=2, C=3)
    tiles = workloads.draw_tiles(w)
    compare.assert_bitexact(oracle.blend_workload(w, tiles), tiles[0], dtype, "1x1")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("ndim", [4, 5])
def test_zero_blend_extent_is_crop_and_concatenate(dtype, ndim):
    if ndim == 4:
        w = _wl(dtype, [20, 20, 9], [20, 20, 20, 5], 0, 14)
    else:
        w = _wl(dtype, [20, 9], [20, 7], 0, 14, ndim=5, ext_t=(6, 6, 2), Et=0, Rt=4)
    tiles = workloads.draw_tiles(w)
    nt, nh, nw = w.grid
    chunks = []
    k = 0
    for tau in range(nt):
        rows = []
        for i in range(nh):
            row = []
            for j in range(nw):
                t = tiles[k].reshape(w.N, w.C, w.ext_t[tau], w.ext_h[i], w.ext_w[j])
                k += 1
                ct = w.row_limit[0] if tau < nt - 1 else w.ext_t[tau]
                ch = w.row_limit[1] if i < nh - 1 else w.ext_h[i]
                cw = w.row_limit[2] if j < nw - 1 else w.ext_w[j]
                row.append(t[:, :, :ct, :ch, :cw])
            rows.append(np.concatenate(row, axis=4))
        chunks.append(np.concatenate(rows, axis=3))
    want = np.concatenate(chunks, axis=2)
    if ndim == 4:
        want = want[:, :, 0]
    compare.assert_bitexact(oracle.blend_workload(w, tiles), want, dtype, "E=0")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_single_row_of_tiles_only_blends_along_w(dtype):
    # n_h = 1: the first seam column equals the left tile's tail exactly (w=0),
    # rows are independent, and the H blend extent is irrelevant
    w1 = _wl(dtype, [21], [30, 30, 12], 10, 20)
    w2 = dataclasses.replace(w1, blend=(0, 0, 10))
    tiles = workloads.draw_tiles(w1)
    o1, o2 = oracle.blend_workload(w1, tiles), oracle.blend_workload(w2, tiles)
    compare.assert_bitexact(o1, o2, dtype, "n_h=1")
    left = tiles[0].reshape(1, 2, 21, 30)
    compare.assert_bitexact(np.ascontiguousarray(o1[..., 20]), np.ascontiguousarray(left[..., 20]), dtype, "w0 col")


def test_extent_clamp_at_sliver():
    # a 6-wide last tile with E = 16 blends over e = 6, with weights k/6
    w = _wl("fp32", [10], [40, 40, 6], 16, 24)
    tiles = workloads.draw_tiles(w)
    out = oracle.blend_workload(w, tiles)
    a = tiles[1].reshape(1, 2, 10, 40)[..., 34:40]
    b = tiles[2].reshape(1, 2, 10, 6)
    wa, wb = models.coeff_f32(6)
    want = (a * wa).astype(np.float32) + (b * wb).astype(np.float32)
    assert np.array_equal(out[..., 48:54], want.astype(np.float32))


# ---------------------------------------------------------------------------
# brute force on tiny grids: three implementations that share no code
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("ndim", [4, 5])
def test_oracle_equals_literal_torch_and_closed_form(dtype, ndim):
    for seed in range(12):
        w = workloads.random_blend_workload(100 + seed, dtype, ndim=ndim)
        tiles = workloads.draw_tiles(w)
        o = oracle.blend_workload(w, tiles)
        compare.assert_bitexact(models.literal_torch(w, tiles), o, dtype, f"literal {w}")
        compare.assert_bitexact(models.closed_form_numpy(w, tiles), o, dtype, f"closed form {w}")


def test_config1_three_ways():
    w, tiles = workloads.draw_config_blend(1)
    o = oracle.blend_workload(w, tiles)
    compare.assert_bitexact(models.literal_torch(w, tiles), o, "fp32", "cfg1 literal")
    compare.assert_bitexact(models.closed_form_numpy(w, tiles), o, "fp32", "cfg1 closed")


def test_in_place_order_matters_and_oracle_uses_it():
    # reading the original (unblended) neighbour instead of the one blended in
    # place changes the corner values: the pins can tell the two apart
    w = _wl("fp16", [30, 30], [30, 30], 12, 18)
    tiles = workloads.draw_tiles(w)
    o = oracle.blend_workload(w, tiles)
    wrong = models.literal_torch(w, tiles, in_place=False)
    assert compare.bit_mismatches(wrong, o, "fp16").size > 0
    compare.assert_bitexact(models.literal_torch(w, tiles), o, "fp16", "in place")


def test_temporal_blend_comes_after_spatial_stitch():
    w = _wl("bf16", [30, 30], [30, 30], 12, 18, ndim=5, ext_t=(9, 9, 9), Et=4, Rt=5, seed=4)
    tiles = workloads.draw_tiles(w)
    o = oracle.blend_workload(w, tiles)
    wrong = models.literal_torch(w, tiles, temporal_first=True)
    assert compare.bit_mismatches(wrong, o, "bf16").size > 0
    compare.assert_bitexact(models.literal_torch(w, tiles), o, "bf16", "spatial first")


# ---------------------------------------------------------------------------
# the comparator itself must reject near-misses
# ---------------------------------------------------------------------------
def test_comparator_rejects_one_ulp_swap_and_zero_sign():
    w, tiles = workloads.draw_config_blend(1)
    o = oracle.blend_workload(w, tiles)
    flip = o.copy()
    flip.view(np.uint32)[0, 1, 50, 60] ^= 1
    assert compare.bit_mismatches(flip, o, "fp32").size == 1
    sw = list(tiles)
    sw[1], sw[2] = sw[2], sw[1]
    assert compare.bit_mismatches(oracle.blend_workload(w, sw), o, "fp32").size > 0
    z = np.zeros(4, np.float32)
    nz = -z
    assert compare.bit_mismatches(z, nz, "fp32").size == 4
    with pytest.raises(AssertionError):
        compare.assert_bitexact(flip, o, "fp32")
