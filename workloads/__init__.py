"""Seeded synthetic workloads shared by the oracle side and the HIP side.

This module only describes inputs: tile-grid extents, sizes, seeds and value
distributions, and draws the input arrays.  It holds none of the method's
arithmetic (no blend extents, crops, coefficients, statistics or outputs); each
side derives those on its own from the numbers returned here.

Arrays are returned as numpy arrays in *storage* form:
  fp32 -> numpy.float32, fp16 -> numpy.float16, bf16 -> numpy.uint16 (raw bits).

Recipe (every config): ``numpy.random.default_rng(seed)``; values drawn in
float64, converted to float32 and then rounded to nearest-even into the storage
dtype (torch's CPU conversion is used for that input rounding).  Draw order:
blend tiles in raster order (temporal tile, tile row, tile column), then the
GroupNorm per-patch offsets, x, gamma, beta.

Workload shapes follow the five configurations of the tiled-VAE assembly
benchmark (with the readings taken where the pages are
silent): a 112x112 fp32 toy, an SD-v1-size 1024x1024 fp16 decode, a 2048x2048
bf16 decode plus a decoder-intermediate GroupNorm, a 49-frame 480x832 bf16
video decode plus a 5-D GroupNorm, and a 4096x4096 fp16 batch-2 decode with
edge slivers plus an fp16 GroupNorm split along W.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")
DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}
ITEMSIZE = {"fp32": 4, "fp16": 2, "bf16": 2}


# ----------------------------------------------------------------------------
# tile layouts (inputs to both sides: how many tiles and how long each is)
# ----------------------------------------------------------------------------
def stock_layout(length: int, tile: int, stride: int) -> List[int]:
    """Stock tiled-decode layout: a tile starts at every multiple of the stride
    below the canvas length; the last one is cut short by the canvas edge (the
    "edge sliver")."""
    if length <= 0 or tile <= 0 or stride <= 0:
        raise ValueError("length, tile and stride must be positive")
    return [min(tile, length - k) for k in range(0, length, stride)]


def fixed_count_layout(count: int, tile: int) -> List[int]:
    """A stated number of equal, full-size tiles (the last one ends at the
    canvas edge at full size)."""
    return [tile] * count


@dataclasses.dataclass(frozen=True)
class BlendWorkload:
    name: str
    dtype: str
    ndim: int                 # 4 (N,C,H,W) or 5 (N,C,T,H,W)
    N: int
    C: int
    ext_t: Sequence[int]      # per temporal tile frame counts ([1] for 4-D)
    ext_h: Sequence[int]
    ext_w: Sequence[int]
    blend: Sequence[int]      # (E_t, E_h, E_w)
    row_limit: Sequence[int]  # (R_t, R_h, R_w)
    seed: int
    std: float = 0.5
    clamp: Optional[float] = None

    @property
    def grid(self):
        return (len(self.ext_t), len(self.ext_h), len(self.ext_w))

    @property
    def n_tiles(self):
        a, b, c = self.grid
        return a * b * c

    def tile_shape(self, tau: int, i: int, j: int):
        if self.ndim == 4:
            return (self.N, self.C, self.ext_h[i], self.ext_w[j])
        return (self.N, self.C, self.ext_t[tau], self.ext_h[i], self.ext_w[j])

    def tile_elems(self) -> int:
        return self.N * self.C * sum(self.ext_t) * sum(self.ext_h) * sum(self.ext_w)


@dataclasses.dataclass(frozen=True)
class GroupNormWorkload:
    name: str
    dtype: str
    shape: Sequence[int]
    groups: int
    split_axis: int
    n_patches: int
    eps: float
    seed: int
    # per-patch mean offset: ("fixed", [o_0, ..]) or ("uniform", lo, hi) or None
    offset: Optional[tuple] = None
    affine: bool = True

    def numel(self) -> int:
        return int(np.prod(self.shape))


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    title: str
    blend: Optional[BlendWorkload]
    groupnorm: Optional[GroupNormWorkload]


def _cfg1():
    b = BlendWorkload("cfg1-blend-112-fp32", "fp32", 4, 1, 3, [1],
                      fixed_count_layout(2, 64), fixed_count_layout(2, 64),
                      (0, 16, 16), (1, 48, 48), seed=1, clamp=None)
    g = GroupNormWorkload("cfg1-gn-fp32", "fp32", (1, 32, 32, 32), 8, 2, 2, 1e-6,
                          seed=1, offset=("fixed", [0.0, 3.0]))
    return Config(1, "fp32 toy: 2x2 tiles -> 112x112; GroupNorm [1,32,32,32]", b, g)


def _cfg2():
    b = BlendWorkload("cfg2-blend-1024-fp16", "fp16", 4, 1, 3, [1],
                      stock_layout(1024, 512, 384), stock_layout(1024, 512, 384),
                      (0, 128, 128), (1, 384, 384), seed=2, clamp=1.0)
    return Config(2, "SD-v1-size 1024x1024 fp16 decode assembly", b, None)


def _cfg3():
    b = BlendWorkload("cfg3-blend-2048-bf16", "bf16", 4, 1, 3, [1],
                      fixed_count_layout(5, 512), fixed_count_layout(5, 512),
                      (0, 128, 128), (1, 384, 384), seed=3, clamp=1.0)
    g = GroupNormWorkload("cfg3-gn-bf16", "bf16", (1, 512, 256, 256), 32, 2, 4, 1e-6,
                          seed=3, offset=("uniform", -2.0, 2.0))
    return Config(3, "2048x2048 bf16 decode + GroupNorm [1,512,256,256]", b, g)


def _cfg4():
    b = BlendWorkload("cfg4-blend-video-bf16", "bf16", 5, 1, 3,
                      stock_layout(49, 17, 12), stock_layout(480, 256, 192),
                      stock_layout(832, 256, 192),
                      (5, 64, 64), (12, 192, 192), seed=4, clamp=1.0)
    g = GroupNormWorkload("cfg4-gn-video-bf16", "bf16", (1, 128, 13, 60, 104), 32, 3, 4,
                          1e-6, seed=4, offset=("uniform", -2.0, 2.0))
    return Config(4, "49x480x832 bf16 video decode + 5-D GroupNorm", b, g)


def _cfg5():
    b = BlendWorkload("cfg5-blend-4096-fp16", "fp16", 4, 2, 3, [1],
                      stock_layout(4096, 576, 448), stock_layout(4096, 576, 448),
                      (0, 128, 128), (1, 448, 448), seed=5, clamp=None)
    g = GroupNormWorkload("cfg5-gn-fp16", "fp16", (2, 256, 512, 512), 32, 3, 8, 1e-6,
                          seed=5, offset=("uniform", -2.0, 2.0))
    return Config(5, "4096x4096 fp16 batch-2 decode with slivers + GroupNorm split on W", b, g)


CONFIGS = {c.index: c for c in (_cfg1(), _cfg2(), _cfg3(), _cfg4(), _cfg5())}


# ----------------------------------------------------------------------------
# drawing values
# ----------------------------------------------------------------------------
def to_storage(values_f64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 -> storage dtype, rounding to nearest even."""
    f32 = np.ascontiguousarray(values_f64, dtype=np.float32)
    if dtype == "fp32":
        return f32
    if dtype == "fp16":
        return f32.astype(np.float16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def storage_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of storage values to float64 (for reporting only)."""
    if dtype in ("fp32", "fp16"):
        return arr.astype(np.float64)
    bits = arr.astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def draw_tiles(w: BlendWorkload, rng: Optional[np.random.Generator] = None):
    """Tiles in raster order (tau, i, j); each N(0, std), optionally clamped."""
    rng = rng if rng is not None else np.random.default_rng(w.seed)
    out = []
    nt, nh, nw = w.grid
    for tau in range(nt):
        for i in range(nh):
            for j in range(nw):
                v = rng.normal(0.0, w.std, size=w.tile_shape(tau, i, j))
                if w.clamp is not None:
                    np.clip(v, -w.clamp, w.clamp, out=v)
                out.append(to_storage(v, w.dtype))
    return out


def patch_bounds(length: int, n_patches: int):
    """array_split convention for the patch split: the first (length mod P)
    patches are one longer.  Returned as a list of (start, stop)."""
    base, extra = divmod(length, n_patches)
    bounds, s = [], 0
    for p in range(n_patches):
        n = base + (1 if p < extra else 0)
        bounds.append((s, s + n))
        s += n
    return bounds


def draw_groupnorm(g: GroupNormWorkload, rng: Optional[np.random.Generator] = None):
    """(x, gamma, beta) in storage form.  x ~ N(0,1) plus a per-patch offset
    shared over N and C; gamma ~ N(1, 0.1), beta ~ N(0, 0.1) (None if no affine)."""
    rng = rng if rng is not None else np.random.default_rng(g.seed)
    offs = None
    if g.offset is not None:
        if g.offset[0] == "fixed":
            offs = np.asarray(g.offset[1], dtype=np.float64)
        else:
            offs = rng.uniform(g.offset[1], g.offset[2], size=g.n_patches)
    x = rng.normal(0.0, 1.0, size=tuple(g.shape))
    if offs is not None:
        L = g.shape[g.split_axis]
        for p, (s, e) in enumerate(patch_bounds(L, g.n_patches)):
            idx = [slice(None)] * len(g.shape)
            idx[g.split_axis] = slice(s, e)
            x[tuple(idx)] += offs[p]
    C = g.shape[1]
    gamma = beta = None
    if g.affine:
        gamma = to_storage(rng.normal(1.0, 0.1, size=C), g.dtype)
        beta = to_storage(rng.normal(0.0, 0.1, size=C), g.dtype)
    return to_storage(x, g.dtype), gamma, beta


def draw_config_blend(index: int):
    w = CONFIGS[index].blend
    return w, draw_tiles(w)


def draw_config_groupnorm(index: int):
    """GroupNorm inputs of a config, drawn after that config's tiles so the
    stream matches the stated draw order."""
    cfg = CONFIGS[index]
    rng = np.random.default_rng(cfg.groupnorm.seed)
    if cfg.blend is not None:
        # advance the stream past the tiles without materialising them
        w = cfg.blend
        nt, nh, nw = w.grid
        for tau in range(nt):
            for i in range(nh):
                for j in range(nw):
                    rng.normal(0.0, w.std, size=w.tile_shape(tau, i, j))
    return cfg.groupnorm, draw_groupnorm(cfg.groupnorm, rng)


# ----------------------------------------------------------------------------
# random small geometries for property and parity tests
# ----------------------------------------------------------------------------
def random_blend_workload(seed: int, dtype: str, ndim: int = 4, max_tiles: int = 4,
                          max_ext: int = 40, align: int = 1, N: int = 1, C: int = 2,
                          std: float = 0.5) -> BlendWorkload:
    """A random tile grid that satisfies the data-parallel preconditions:
    every non-last tile is at least the row limit long, and every tile is at
    least as long as the blend extents on its two sides together.  `align`
    makes every W extent, W row limit and W blend extent a multiple of it."""
    rng = np.random.default_rng(seed)

    def axis(max_n, max_len, a):
        n = int(rng.integers(1, max_n + 1))
        E = int(rng.integers(0, max(2, max_len // 2))) // a * a
        R = int(rng.integers(1, max_len)) // a * a
        R = max(R, a)
        T = R + E  # stock tiles: stride + blend
        exts = []
        for k in range(n):
            if k < n - 1:
                exts.append(T)
            else:
                exts.append(max(a, int(rng.integers(1, T + 1)) // a * a))
        # enforce ext(k) >= e(k) + e(k+1) by construction: shrink E if needed
        def ok(Ev):
            es = [0] + [min(Ev, exts[k - 1], exts[k]) for k in range(1, n)] + [0]
            return all(exts[k] >= es[k] + es[k + 1] for k in range(n))
        while E > 0 and not ok(E):
            E -= a
        return n, exts, E, R

    nt_max = max_tiles if ndim == 5 else 1
    if ndim == 5:
        nt, et, Et, Rt = axis(nt_max, max(4, max_ext // 4), 1)
    else:
        nt, et, Et, Rt = 1, [1], 0, 1
    nh, eh, Eh, Rh = axis(max_tiles, max_ext, 1)
    nw, ew, Ew, Rw = axis(max_tiles, max_ext, align)
    return BlendWorkload(f"random-{seed}-{dtype}-{ndim}d", dtype, ndim, N, C, et, eh, ew,
                         (Et, Eh, Ew), (Rt, Rh, Rw), seed=seed, std=std)


# ----------------------------------------------------------------------------
# wide tiles blended with the normalised ramp (decode in pixels, encode in
# latents); origins and extents are stated as numbers, margins and ramps in
# positions (latents times the VAE's compression ratio for decoded pixels)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class RampWorkload:
    name: str
    dtype: str
    lead: Sequence[int]        # (N, C) or (N, C, T)
    origins_h: Sequence[int]
    extents_h: Sequence[int]
    origins_w: Sequence[int]
    extents_w: Sequence[int]
    margin: Sequence[int]      # (h, w)
    ramp: Sequence[int]        # (h, w)
    seed: int
    std: float = 0.5
    clamp: Optional[float] = 1.0

    @property
    def out_shape(self):
        LH = max(o + e for o, e in zip(self.origins_h, self.extents_h))
        LW = max(o + e for o, e in zip(self.origins_w, self.extents_w))
        return tuple(self.lead) + (LH, LW)

    def tile_shape(self, i: int, j: int):
        return tuple(self.lead) + (self.extents_h[i], self.extents_w[j])


def _scaled(latents: Sequence[int], ratio: int) -> List[int]:
    return [int(v) * ratio for v in latents]


# Qwen-Image-2.1 (16x): 2048 px = 128 latents in the 32-latent floor tiles with
# 16-latent overlaps, spread evenly: origins 0, 16, ..., 96 latents.
_Q21_2048 = list(range(0, 97, 16))
# Qwen-Image-2.1 at 2752x1536 px: 172 x 96 latents, floor tiles spread evenly
_Q21_2752_W = [0, 15, 31, 46, 62, 77, 93, 108, 124, 140]
_Q21_1536_H = [0, 16, 32, 48, 64]

RAMP_WORKLOADS = {
    # decode, pixel space: margin 4 latents and ramp 8 latents times the ratio
    "qwen21-2048-bf16": RampWorkload(
        "qwen21-2048-bf16", "bf16", (1, 3), _scaled(_Q21_2048, 16), [512] * 7,
        _scaled(_Q21_2048, 16), [512] * 7, (64, 64), (128, 128), seed=21),
    "qwen21-2752x1536-bf16": RampWorkload(
        "qwen21-2752x1536-bf16", "bf16", (1, 3, 1), _scaled(_Q21_1536_H, 16), [512] * 5,
        _scaled(_Q21_2752_W, 16), [512] * 10, (64, 64), (128, 128), seed=22),
    # FLUX.1 (8x) at 1600 px: two 120-latent tiles per side at 0 and 80 latents
    "flux-1600-bf16": RampWorkload(
        "flux-1600-bf16", "bf16", (1, 3), [0, 640], [960, 960], [0, 640], [960, 960],
        (32, 32), (64, 64), seed=23),
    # encode, latent space: 64-latent tiles with 32-latent overlaps, the
    # decode's margin and ramp in latents; 16 latent channels; a 2048 px
    # reference at 16x is 128 latents
    "qwen21-encode-2048-bf16": RampWorkload(
        "qwen21-encode-2048-bf16", "bf16", (1, 16), [0, 32, 64], [64] * 3, [0, 32, 64], [64] * 3,
        (4, 4), (8, 8), seed=24, std=1.0, clamp=None),
}


# Stock tiled encode of an SD-class AutoencoderKL (8x, 4 latent channels): 512 px
# sample tiles at a 384 px stride give 64-latent tiles every 48 latents, blended
# over 16 latents; a 2048 px image is 256 latents, the last tile a 16-latent sliver.
# Also the 64-latent tiles with 32-latent overlaps of the wide-tile encode.
ENCODE_BLEND_WORKLOADS = {
    "sd-encode-2048-fp16": BlendWorkload(
        "sd-encode-2048-fp16", "fp16", 4, 1, 4, [1], stock_layout(256, 64, 48),
        stock_layout(256, 64, 48), (0, 16, 16), (1, 48, 48), seed=25, std=1.0, clamp=None),
    # the same blend on 16-channel latents in 64-latent tiles with 32-latent
    # overlaps (the wide-tile encode geometry), stock placement: 128 latents
    "encode-64-32-2048-bf16": BlendWorkload(
        "encode-64-32-2048-bf16", "bf16", 4, 1, 16, [1], stock_layout(128, 64, 32),
        stock_layout(128, 64, 32), (0, 32, 32), (1, 32, 32), seed=27, std=1.0, clamp=None),
    "sd-encode-4096-bf16-batch4": BlendWorkload(
        "sd-encode-4096-bf16-batch4", "bf16", 4, 4, 4, [1], stock_layout(512, 64, 48),
        stock_layout(512, 64, 48), (0, 16, 16), (1, 48, 48), seed=26, std=1.0, clamp=None),
}


def draw_ramp_tiles(w: RampWorkload, rng: Optional[np.random.Generator] = None):
    """Tiles in raster order (i, j); each N(0, std), optionally clamped."""
    rng = rng if rng is not None else np.random.default_rng(w.seed)
    out = []
    for i in range(len(w.origins_h)):
        for j in range(len(w.origins_w)):
            v = rng.normal(0.0, w.std, size=w.tile_shape(i, j))
            if w.clamp is not None:
                np.clip(v, -w.clamp, w.clamp, out=v)
            out.append(to_storage(v, w.dtype))
    return out


def random_ramp_workload(seed: int, dtype: str, lead=(1, 2), max_tiles: int = 4, max_ext: int = 48,
                         align: int = 1) -> RampWorkload:
    """Random increasing origins and extents with every tile inside the canvas,
    overlaps wide enough for a tile with weight everywhere (more than twice the
    margin plus one), and `align` dividing every W origin and extent."""
    rng = np.random.default_rng(seed)

    def axis(a):
        m = int(rng.integers(0, 5))
        r = int(rng.integers(1, 9))
        n = int(rng.integers(1, max_tiles + 1))
        s = max(2 * m + 2 + a, int(rng.integers(2 * m + 2, max_ext + 1)))
        s = -(-s // a) * a
        origins, extents = [0], [s]
        for k in range(1, n):
            ov_min = 2 * m + 2
            stride = int(rng.integers(1, max(2, s - ov_min + 1)))
            stride = max(a, stride // a * a)
            if s - stride < ov_min:
                break
            origins.append(origins[-1] + stride)
            extents.append(s)
        return origins, extents, m, r

    oh, eh, mh, rh = axis(1)
    ow, ew, mw, rw = axis(align)
    return RampWorkload(f"ramp-random-{seed}-{dtype}", dtype, tuple(lead), oh, eh, ow, ew,
                        (mh, mw), (rh, rw), seed=seed, clamp=None)
