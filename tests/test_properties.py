"""Property tests over generated tiny geometries (hypothesis): the blend
oracle against two independent brute-force models, the layout planner against
its search oracle, and the ramp oracle against a factored per-axis
normalisation.  CPU only."""
from __future__ import annotations

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import compare
import models
import oracle
import workloads
from oracle import layout as ol

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def blend_grids(draw):
    """A tiny tile grid meeting the closed form's preconditions: slivers,
    clamped extents, 1xN grids, E = 0 and 5-D included."""
    dtype = draw(st.sampled_from(["fp32", "fp16", "bf16"]))
    ndim = draw(st.sampled_from([4, 5]))

    def axis(max_n, max_r):
        n = draw(st.integers(1, max_n))
        R = draw(st.integers(1, max_r))
        E = draw(st.integers(0, max_r))
        exts = [R + draw(st.integers(0, E)) for _ in range(n - 1)]
        exts.append(draw(st.integers(1, R + E)))
        # clamp E until every tile holds its two seams
        while E > 0:
            es = [0] + [min(E, exts[k - 1], exts[k]) for k in range(1, n)] + [0]
            if all(exts[k] >= es[k] + es[k + 1] for k in range(n)):
                break
            E -= 1
        return exts, E, R

    et, Et, Rt = axis(3, 4) if ndim == 5 else ([1], 0, 1)
    eh, Eh, Rh = axis(3, 7)
    ew, Ew, Rw = axis(3, 7)
    N = draw(st.integers(1, 2))
    C = draw(st.integers(1, 2))
    seed = draw(st.integers(0, 2**31 - 1))
    return workloads.BlendWorkload("hyp", dtype, ndim, N, C, et, eh, ew, (Et, Eh, Ew), (Rt, Rh, Rw),
                                   seed=seed)


@SETTINGS
@given(blend_grids())
def test_blend_oracle_equals_literal_and_closed_form_models(w):
    tiles = workloads.draw_tiles(w)
    o = oracle.blend_workload(w, tiles)
    compare.assert_bitexact(models.literal_torch(w, tiles), o, w.dtype, f"literal {w}")
    compare.assert_bitexact(models.closed_form_numpy(w, tiles), o, w.dtype, f"closed form {w}")


@pytest.fixture(scope="module")
def sb():
    import seam_blending_patch_amd as m
    return m


@st.composite
def layouts(draw):
    rule = draw(st.sampled_from(["stock", "edge_aligned", "fewest_calls", "smallest_side", "auto"]))
    L = draw(st.integers(1, 600))
    T = draw(st.integers(1, 200))
    S = draw(st.integers(1, T))
    ov = draw(st.integers(0, max(0, T - 4)))
    M = draw(st.integers(ov + 4, ov + 250))
    ov_e = draw(st.integers(0, T + 4))  # may reach the tile side: valid only for one tile
    p = {"stock": [T, S], "edge_aligned": [T, ov_e], "fewest_calls": [T, S, ov, M],
         "smallest_side": [ov, M],
         "auto": [T, S, draw(st.integers(1, 64)), draw(st.integers(0, 32))]}[rule]
    return L, rule, p


@SETTINGS
@given(layouts())
def test_planner_equals_search_oracle(sb, case):
    L, rule, p = case
    try:
        want = ol.layout(L, rule, p)
    except ValueError:
        with pytest.raises(sb.SeamBlendError):
            sb.vae_tile_layout(L, rule, p)
        return
    o, e = sb.vae_tile_layout(L, rule, p)
    assert list(zip(o, e)) == want
    assert ol.covers(L, want, 0)


@st.composite
def ramp_layouts(draw):
    def axis():
        m = draw(st.integers(0, 3))
        r = draw(st.integers(1, 6))
        s = draw(st.integers(2 * m + 3, 24))
        n = draw(st.integers(1, 3))
        origins = [0]
        for _ in range(n - 1):
            stride = draw(st.integers(1, s - (2 * m + 2)))
            origins.append(origins[-1] + stride)
        return origins, [s] * len(origins), m, r

    oh, eh, mh, rh = axis()
    ow, ew, mw, rw = axis()
    return workloads.RampWorkload("hyp", "fp32", (1, 2), oh, eh, ow, ew, (mh, mw), (rh, rw),
                                  seed=draw(st.integers(0, 2**31 - 1)), clamp=None)


@SETTINGS
@given(ramp_layouts())
def test_ramp_oracle_equals_factored_normalisation(w):
    tiles = workloads.draw_ramp_tiles(w)
    ref = oracle.ramp_blend(tiles, w.lead, w.origins_h, w.extents_h, w.origins_w, w.extents_w,
                            w.margin, w.ramp, "fp32")

    def table(origins, extents, m, r, L):
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

    LH, LW = ref.shape[-2:]
    th = table(w.origins_h, w.extents_h, w.margin[0], w.ramp[0], LH)
    tw = table(w.origins_w, w.extents_w, w.margin[1], w.ramp[1], LW)
    acc = np.zeros(ref.shape)
    nw = len(w.origins_w)
    for i, (oh, sh) in enumerate(zip(w.origins_h, w.extents_h)):
        for j, (ow, sw) in enumerate(zip(w.origins_w, w.extents_w)):
            acc[..., oh:oh + sh, ow:ow + sw] += (th[i, oh:oh + sh, None] * tw[j, None, ow:ow + sw]
                                                 * tiles[i * nw + j].astype(np.float64))
    assert np.max(np.abs(acc - ref)) < 1e-12
