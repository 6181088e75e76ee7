"""MI355X (gfx950) tiled-VAE decode assembly: blend + crop + stitch of
overlapping decoded tiles, and patch-split GroupNorm.

This module is the thin Python binding of ``libseamblend.so`` (C ABI in
``include/seam_blend.h``): it turns torch tensors into pointers, sizes and the
current HIP stream and calls the library.  PyTorch is used for device memory
and streams only; every step of both operations runs in the library's HIP
kernels.  There is no CPU fallback: importing this package fails if the
library has not been built, and every call requires GPU tensors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import torch

__all__ = ["vae_tile_layout", "LAYOUT_RULES", "vae_tile_ramp_blend", "RampBlend", "vae_tile_blend_stitch", "vae_tile_blend_stitch_output_extents", "BlendStitch",
           "patch_groupnorm", "patch_groupnorm_workspace_bytes", "PatchGroupNorm",
           "patch_groupnorm_noalloc", "GN_STATIC_SCRATCH_BYTES",
           "SeamBlendError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libseamblend.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python seam_blending_patch_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)
_i64p = ctypes.POINTER(ctypes.c_int64)
_lib.vae_tile_blend_stitch_output_extents.argtypes = [_i64p, _i64p, _i64p, _i64p, _i64p]
_lib.vae_tile_blend_stitch_output_extents.restype = ctypes.c_int
_lib.vae_tile_blend_stitch.argtypes = [ctypes.POINTER(ctypes.c_void_p), _i64p, _i64p, _i64p, _i64p,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
_lib.vae_tile_blend_stitch.restype = ctypes.c_int
_lib.patch_groupnorm_workspace_bytes.argtypes = [ctypes.c_int, _i64p, ctypes.c_int64, ctypes.c_int,
                                                 ctypes.c_int64]
_lib.patch_groupnorm_workspace_bytes.restype = ctypes.c_size_t
_lib.patch_groupnorm.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p, ctypes.c_void_p]
_lib.patch_groupnorm.restype = ctypes.c_int
_lib.patch_groupnorm_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64p, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.patch_groupnorm_noalloc.restype = ctypes.c_int
_lib.vae_tile_layout.argtypes = [ctypes.c_int64, ctypes.c_int, _i64p, ctypes.c_int64, _i64p, _i64p, _i64p]
_lib.vae_tile_layout.restype = ctypes.c_int
_lib.vae_tile_ramp_blend.argtypes = [ctypes.POINTER(ctypes.c_void_p), _i64p, _i64p, _i64p, _i64p, _i64p,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
_lib.vae_tile_ramp_blend.restype = ctypes.c_int
_lib.seamblend_last_error.argtypes = []
_lib.seamblend_last_error.restype = ctypes.c_char_p

_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class SeamBlendError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.seamblend_last_error().decode(errors="replace")
        super().__init__(f"{where} failed ({code}): {msg}")
        self.code = code


def _arr(vals: Sequence[int]):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _check(rc: int, where: str):
    if rc != 0:
        raise SeamBlendError(rc, where)


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require_gpu(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in _DTYPE:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}")


def _triple(v, name):
    if isinstance(v, int):
        return (v, v, v)
    v = tuple(int(a) for a in v)
    if len(v) == 2:
        return (0,) + v
    if len(v) != 3:
        raise ValueError(f"{name} must be an int, (h, w) or (t, h, w)")
    return v


def _grid_of(tiles):
    """Nested tiles -> (ndim, flat list in raster order, n_t, n_h, n_w)."""
    first = tiles[0][0]
    if isinstance(first, torch.Tensor):  # [i][j] of 4-D tiles
        grid3 = [tiles]
    else:
        grid3 = tiles
    flat = [t for plane in grid3 for row in plane for t in row]
    nt, nh, nw = len(grid3), len(grid3[0]), len(grid3[0][0])
    for plane in grid3:
        if len(plane) != nh or any(len(r) != nw for r in plane):
            raise ValueError("tile grid is ragged")
    ndim = flat[0].dim()
    if ndim not in (4, 5) or (ndim == 4 and nt != 1) or any(t.dim() != ndim for t in flat):
        raise ValueError("tiles must be 4-D [N,C,h,w] in an [i][j] grid or 5-D [N,C,t,h,w] in [tau][i][j]")
    return ndim, grid3, flat, nt, nh, nw


def _extents(grid3, ndim, nt, nh, nw):
    t0 = grid3[0][0][0]
    N, C = t0.shape[0], t0.shape[1]
    et = [grid3[tau][0][0].shape[2] if ndim == 5 else 1 for tau in range(nt)]
    eh = [grid3[0][i][0].shape[-2] for i in range(nh)]
    ew = [grid3[0][0][j].shape[-1] for j in range(nw)]
    for tau in range(nt):
        for i in range(nh):
            for j in range(nw):
                t = grid3[tau][i][j]
                want = (N, C, et[tau], eh[i], ew[j]) if ndim == 5 else (N, C, eh[i], ew[j])
                if tuple(t.shape) != want:
                    raise ValueError(f"tile ({tau},{i},{j}) has shape {tuple(t.shape)}, expected {want}")
    return N, C, et, eh, ew


LAYOUT_RULES = {"stock": 0, "edge_aligned": 1, "fewest_calls": 2, "smallest_side": 3, "auto": 4}


def vae_tile_layout(length: int, rule: str, params: Sequence[int], max_tiles: int = 4096):
    """Tile layout along one axis (host-side): (origins, extents) lists.  Rules
    and params as in ``include/seam_blend.h`` (``vae_tile_layout``)."""
    p = list(params) + [0] * (4 - len(params))
    o = (ctypes.c_int64 * max_tiles)()
    e = (ctypes.c_int64 * max_tiles)()
    n = ctypes.c_int64(0)
    _check(_lib.vae_tile_layout(int(length), LAYOUT_RULES[rule], _arr(p), max_tiles, o, e,
                                ctypes.byref(n)), "vae_tile_layout")
    return list(o[: n.value]), list(e[: n.value])


def vae_tile_blend_stitch_output_extents(grid: Sequence[int], tile_extents: Sequence[int],
                                         blend_extent: Sequence[int], row_limit: Sequence[int]):
    """(L_t, L_h, L_w) of the stitched output (host-only validation)."""
    out = (ctypes.c_int64 * 3)()
    _check(_lib.vae_tile_blend_stitch_output_extents(_arr(grid), _arr(tile_extents),
                                                     _arr(blend_extent), _arr(row_limit), out),
           "vae_tile_blend_stitch_output_extents")
    return tuple(out)


class BlendStitch:
    """A prepared blend + crop + stitch call: validates the tile grid and builds
    the C arguments once; each call enqueues the kernel on the current stream.

    tiles: ``tiles[i][j]`` 4-D ``[N,C,h_i,w_j]`` or ``tiles[tau][i][j]`` 5-D
    ``[N,C,t_tau,h_i,w_j]`` contiguous GPU tensors of one dtype (fp32, fp16,
    bf16).  blend_extent / row_limit: int, (h, w) or (t, h, w).  The call reads
    the tiles' current contents, so the same object can be replayed after the
    tiles are refilled (the tensors must stay alive and in place).
    """

    def __init__(self, tiles, blend_extent, row_limit, out: Optional[torch.Tensor] = None):
        ndim, grid3, flat, nt, nh, nw = _grid_of(tiles)
        for k, t in enumerate(flat):
            _require_gpu(t, f"tile {k}")
        dtype, device = flat[0].dtype, flat[0].device
        if any(t.dtype != dtype or t.device != device for t in flat):
            raise ValueError("all tiles must share dtype and device")
        N, C, et, eh, ew = _extents(grid3, ndim, nt, nh, nw)
        E, R = _triple(blend_extent, "blend_extent"), _triple(row_limit, "row_limit")
        if ndim == 4:
            E, R = (0, E[1], E[2]), (1, R[1], R[2])
        grid = (ndim, N, C, nt, nh, nw)
        ext = list(et) + list(eh) + list(ew)
        LT, LH, LW = vae_tile_blend_stitch_output_extents(grid, ext, E, R)
        shape = (N, C, LH, LW) if ndim == 4 else (N, C, LT, LH, LW)
        if out is None:
            out = torch.empty(shape, dtype=dtype, device=device)
        else:
            _require_gpu(out, "out")
            if tuple(out.shape) != shape or out.dtype != dtype or out.device != device:
                raise ValueError(f"out must be {shape} {dtype} on {device}")
        self.out, self.device, self._tiles = out, device, flat
        self._args = ((ctypes.c_void_p * len(flat))(*[t.data_ptr() for t in flat]), _arr(grid),
                      _arr(ext), _arr(E), _arr(R), _DTYPE[dtype], ctypes.c_void_p(out.data_ptr()))

    def __call__(self) -> torch.Tensor:
        rc = _lib.vae_tile_blend_stitch(*self._args, ctypes.c_void_p(_stream_ptr(self.device)))
        if rc != 0:
            raise SeamBlendError(rc, "vae_tile_blend_stitch")
        return self.out


def vae_tile_blend_stitch(tiles, blend_extent: Union[int, Sequence[int]],
                          row_limit: Union[int, Sequence[int]],
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Blend, crop and stitch a grid of decoded tiles on the GPU (see
    BlendStitch).  Returns (or fills) the ``[N,C,(L_t,)L_h,L_w]`` output."""
    plan = BlendStitch(tiles, blend_extent, row_limit, out)
    with torch.cuda.device(plan.device):
        return plan()


def _pair(v, name):
    if isinstance(v, int):
        return (int(v), int(v))
    v = tuple(int(a) for a in v)
    if len(v) != 2:
        raise ValueError(f"{name} must be an int or (h, w)")
    return v


class RampBlend:
    """A prepared normalised-ramp blend of wide tiles (``vae_tile_ramp_blend``).

    tiles: ``tiles[i][j]`` contiguous GPU tensors ``[N,C,h_i,w_j]`` or
    ``[N,C,T,h_i,w_j]`` (frames untiled) of one dtype.  origins_h / origins_w:
    the tiles' row and column origins in positions.  margin / ramp: int or
    (h, w), in positions (for decoded pixels: latents times the VAE's
    compression ratio).  Each call enqueues the kernel on the current stream.
    """

    def __init__(self, tiles, origins_h: Sequence[int], origins_w: Sequence[int],
                 margin: Union[int, Sequence[int]], ramp: Union[int, Sequence[int]],
                 out: Optional[torch.Tensor] = None):
        nh, nw = len(tiles), len(tiles[0])
        if any(len(r) != nw for r in tiles):
            raise ValueError("tile grid is ragged")
        if len(origins_h) != nh or len(origins_w) != nw:
            raise ValueError("one origin per tile row and per tile column")
        flat = [t for row in tiles for t in row]
        for k, t in enumerate(flat):
            _require_gpu(t, f"tile {k}")
        t0 = flat[0]
        ndim, dtype, device = t0.dim(), t0.dtype, t0.device
        if ndim not in (4, 5) or any(t.dim() != ndim or t.dtype != dtype or t.device != device for t in flat):
            raise ValueError("tiles must all be 4-D or all 5-D, of one dtype and device")
        lead = tuple(t0.shape[:-2])
        eh = [tiles[i][0].shape[-2] for i in range(nh)]
        ew = [tiles[0][j].shape[-1] for j in range(nw)]
        for i in range(nh):
            for j in range(nw):
                if tuple(tiles[i][j].shape) != lead + (eh[i], ew[j]):
                    raise ValueError(f"tile ({i},{j}) has shape {tuple(tiles[i][j].shape)}")
        T = lead[2] if ndim == 5 else 1
        LH = max(int(o) + e for o, e in zip(origins_h, eh))
        LW = max(int(o) + e for o, e in zip(origins_w, ew))
        shape = lead + (LH, LW)
        if out is None:
            out = torch.empty(shape, dtype=dtype, device=device)
        else:
            _require_gpu(out, "out")
            if tuple(out.shape) != shape or out.dtype != dtype or out.device != device:
                raise ValueError(f"out must be {shape} {dtype} on {device}")
        m, r = _pair(margin, "margin"), _pair(ramp, "ramp")
        grid = (ndim, lead[0], lead[1], 1, nh, nw)
        self.out, self.device, self._tiles = out, device, flat
        self._args = ((ctypes.c_void_p * len(flat))(*[t.data_ptr() for t in flat]), _arr(grid),
                      _arr([0] + list(origins_h) + list(origins_w)), _arr([T] + eh + ew),
                      _arr((0,) + m), _arr((0,) + r), _DTYPE[dtype], ctypes.c_void_p(out.data_ptr()))

    def __call__(self) -> torch.Tensor:
        rc = _lib.vae_tile_ramp_blend(*self._args, ctypes.c_void_p(_stream_ptr(self.device)))
        if rc != 0:
            raise SeamBlendError(rc, "vae_tile_ramp_blend")
        return self.out


def vae_tile_ramp_blend(tiles, origins_h: Sequence[int], origins_w: Sequence[int],
                        margin: Union[int, Sequence[int]], ramp: Union[int, Sequence[int]],
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Normalised-ramp blend of a grid of wide tiles on the GPU (see RampBlend).
    Returns (or fills) the ``[N,C,(T,)L_h,L_w]`` output."""
    plan = RampBlend(tiles, origins_h, origins_w, margin, ramp, out)
    with torch.cuda.device(plan.device):
        return plan()


def patch_groupnorm_workspace_bytes(shape: Sequence[int], groups: int, split_axis: int,
                                    n_patches: int) -> int:
    n = _lib.patch_groupnorm_workspace_bytes(len(shape), _arr(shape), groups, split_axis, n_patches)
    if n == 0:
        raise SeamBlendError(-1, "patch_groupnorm_workspace_bytes")
    return int(n)


class PatchGroupNorm:
    """A prepared patch GroupNorm call over fixed x / out / gamma / beta
    tensors (arguments validated and the workspace allocated once).  See
    patch_groupnorm for the meaning of the arguments."""

    def __init__(self, x: torch.Tensor, groups: int, split_axis: int, n_patches: int,
                 eps: float = 1e-6, gamma: Optional[torch.Tensor] = None,
                 beta: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 patch_stats: Optional[torch.Tensor] = None):
        _require_gpu(x, "x")
        shape = tuple(x.shape)
        dev = x.device
        for name, t in (("gamma", gamma), ("beta", beta)):
            if t is not None:
                _require_gpu(t, name)
                if t.dtype != x.dtype or t.numel() != shape[1] or t.device != dev:
                    raise ValueError(f"{name} must be [C] of x's dtype on x's device")
        if out is None:
            out = torch.empty_like(x)
        else:
            _require_gpu(out, "out")
            if tuple(out.shape) != shape or out.dtype != x.dtype or out.device != dev:
                raise ValueError("out must match x")
        need = patch_groupnorm_workspace_bytes(shape, groups, split_axis, n_patches)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        elif not workspace.is_cuda or workspace.device != dev:
            raise ValueError("workspace must be a GPU tensor on x's device")
        if patch_stats is not None:
            if (patch_stats.dtype != torch.float32 or not patch_stats.is_cuda
                    or not patch_stats.is_contiguous()
                    or patch_stats.numel() != shape[0] * groups * n_patches * 3):
                raise ValueError("patch_stats must be a contiguous float32 GPU tensor [N, G, P, 3]")
        self.out, self.device = out, dev
        self._keep = (x, gamma, beta, workspace, patch_stats)
        self._args = (ctypes.c_void_p(x.data_ptr()), x.dim(), _arr(shape), groups, split_axis,
                      n_patches, float(eps),
                      ctypes.c_void_p(gamma.data_ptr() if gamma is not None else None),
                      ctypes.c_void_p(beta.data_ptr() if beta is not None else None),
                      _DTYPE[x.dtype], ctypes.c_void_p(out.data_ptr()),
                      ctypes.c_void_p(workspace.data_ptr()),
                      workspace.numel() * workspace.element_size(),
                      ctypes.c_void_p(patch_stats.data_ptr() if patch_stats is not None else None))

    def __call__(self) -> torch.Tensor:
        rc = _lib.patch_groupnorm(*self._args, ctypes.c_void_p(_stream_ptr(self.device)))
        if rc != 0:
            raise SeamBlendError(rc, "patch_groupnorm")
        return self.out


def patch_groupnorm(x: torch.Tensor, groups: int, split_axis: int, n_patches: int,
                    eps: float = 1e-6, gamma: Optional[torch.Tensor] = None,
                    beta: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    patch_stats: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GroupNorm of x ([N,C,...] GPU tensor) from per-patch statistics merged
    with Chan's formula; equals unsplit GroupNorm.  ``out`` may be ``x``.
    ``workspace``: optional uint8 GPU tensor of at least
    ``patch_groupnorm_workspace_bytes`` bytes (allocated here if omitted).
    ``patch_stats``: optional float32 GPU tensor [N, G, P, 3] that receives
    per-patch (count, mean, M2)."""
    plan = PatchGroupNorm(x, groups, split_axis, n_patches, eps, gamma, beta, out, workspace,
                          patch_stats)
    with torch.cuda.device(plan.device):
        return plan()


GN_STATIC_SCRATCH_BYTES = 1 << 20  # SB_GN_STATIC_SCRATCH_BYTES


def patch_groupnorm_noalloc(x: torch.Tensor, groups: int, split_axis: int, n_patches: int,
                            eps: float = 1e-6, gamma: Optional[torch.Tensor] = None,
                            beta: Optional[torch.Tensor] = None, out: torch.Tensor = None,
                            patch_stats: Optional[torch.Tensor] = None) -> torch.Tensor:
    """patch_groupnorm without a workspace: the library keeps the statistics
    in its static per-GPU scratch (problems whose statistics need more than
    GN_STATIC_SCRATCH_BYTES are refused).  ``out`` is required, so that the
    call allocates nothing; calls that overlap on one GPU race."""
    _require_gpu(x, "x")
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    _require_gpu(out, "out")
    if tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype or out.device != x.device:
        raise ValueError("out must match x")
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None:
            _require_gpu(t, name)
            if t.dtype != x.dtype or t.numel() != x.shape[1] or t.device != x.device:
                raise ValueError(f"{name} must be [C] of x's dtype on x's device")
    if patch_stats is not None and (patch_stats.dtype != torch.float32 or not patch_stats.is_cuda
                                    or not patch_stats.is_contiguous()
                                    or patch_stats.numel() != x.shape[0] * groups * n_patches * 3):
        raise ValueError("patch_stats must be a contiguous float32 GPU tensor [N, G, P, 3]")
    with torch.cuda.device(x.device):
        rc = _lib.patch_groupnorm_noalloc(
            ctypes.c_void_p(x.data_ptr()), x.dim(), _arr(x.shape), groups, split_axis, n_patches, float(eps),
            ctypes.c_void_p(gamma.data_ptr() if gamma is not None else None),
            ctypes.c_void_p(beta.data_ptr() if beta is not None else None), _DTYPE[x.dtype],
            ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(patch_stats.data_ptr() if patch_stats is not None else None),
            ctypes.c_void_p(_stream_ptr(x.device)))
    if rc != 0:
        raise SeamBlendError(rc, "patch_groupnorm_noalloc")
    return out
