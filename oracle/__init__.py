"""CPU oracle for tiled-VAE decode assembly and patch-split GroupNorm.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library.  It shares no code
with the HIP path.  The arithmetic lives in ``oracle.c`` (plain C, gcc,
``-ffp-contract=off``); this module only marshals numpy arrays to it.

Functions and the passages they follow:

* ``blend_stitch``  -- literal sequential in-place blend_v / blend_h / blend_t,
  crop to the row limit, stitch (diffusers issue "[Proposal] Vectorize tiled
  VAE blending while preserving rounding and CUDA graph replay", section
  "Proposed scope": clamping, in-place output, per-product rounding, float64
  coefficient division).
* ``groupnorm``     -- unsplit GroupNorm in double (DistVAE PR "Add tiled VAE
  parallelism & extended model support", PatchGroupNorm commit: equal
  nn.GroupNorm, global mean, divide by the count).
* ``ramp_blend``, ``ramp_weight`` -- the normalised-ramp blend of wide tiles
  in double (unsloth Studio PR "size seam-free VAE tiles from measured peaks",
  the Qwen-Image-2.1 wide-tile commit: no weight within the margin of a shared
  edge, a linear ramp over the next positions, weights normalised to 1).
* ``patch_stats``, ``chan_merge`` -- per-patch (count, mean, M2) with the
  Patchify split (first ranks one band longer) and their Chan merge.

Pins: every function here is checked against closed forms, invariants,
library routines and brute force in tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}
NP_STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-shared", "-fPIC", "-Wall", "-Wno-unknown-pragmas"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (a checker, built like any test fixture)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.oracle_blend_stitch.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, i64p, i64p, i64p, ctypes.c_int,
                                          ctypes.c_void_p]
        L.oracle_blend_stitch.restype = ctypes.c_int
        L.oracle_groupnorm.argtypes = [ctypes.c_void_p, ctypes.c_int, i64p, ctypes.c_int64,
                                       ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.oracle_groupnorm.restype = ctypes.c_int
        L.oracle_patch_stats.argtypes = [ctypes.c_void_p, ctypes.c_int, i64p, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_void_p]
        L.oracle_patch_stats.restype = ctypes.c_int
        L.oracle_chan_merge.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p]
        L.oracle_chan_merge.restype = None
        L.oracle_blend_coefficients.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_blend_coefficients.restype = None
        L.oracle_crossfade.argtypes = [ctypes.c_float] * 4 + [ctypes.c_int]
        L.oracle_crossfade.restype = ctypes.c_float
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_ramp_blend.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, i64p, i64p, i64p, i64p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_ramp_blend.restype = ctypes.c_int
        L.oracle_ramp_weight.argtypes = [ctypes.c_int64] * 7
        L.oracle_ramp_weight.restype = ctypes.c_double
        L.oracle_round_f32_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_void_p]
        L.oracle_round_f32_array.restype = None
        L.oracle_widen_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_void_p]
        L.oracle_widen_array.restype = None
        _lib = L
    return _lib


def _i64(seq: Sequence[int]):
    arr = (ctypes.c_int64 * len(seq))(*[int(v) for v in seq])
    return arr


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def output_extents(ext_t, ext_h, ext_w, row_limit):
    """(L_t, L_h, L_w): every tile but the last contributes R, the last its extent."""
    return tuple((len(e) - 1) * int(r) + int(e[-1]) for e, r in zip((ext_t, ext_h, ext_w), row_limit))


def blend_stitch(tiles, N, C, ext_t, ext_h, ext_w, blend, row_limit, dtype, ndim=4):
    """Literal blend + crop + stitch.  ``tiles`` are storage-form numpy arrays in
    raster order (tau, i, j).  Returns the storage-form output of shape
    [N, C, (L_t,) L_h, L_w]."""
    n_t, n_h, n_w = len(ext_t), len(ext_h), len(ext_w)
    assert len(tiles) == n_t * n_h * n_w
    st = NP_STORAGE[dtype]
    keep = [np.ascontiguousarray(t, dtype=st) for t in tiles]
    for k, t in enumerate(keep):
        tau, rem = divmod(k, n_h * n_w)
        i, j = divmod(rem, n_w)
        assert t.size == N * C * ext_t[tau] * ext_h[i] * ext_w[j], "tile size mismatch"
    ptrs = (ctypes.c_void_p * max(1, len(keep)))(*[t.ctypes.data for t in keep])
    LT, LH, LW = output_extents(ext_t, ext_h, ext_w, row_limit)
    shape = (N, C, LH, LW) if ndim == 4 else (N, C, LT, LH, LW)
    if ndim == 4:
        assert n_t == 1 and ext_t[0] == 1
    out = np.zeros(shape, dtype=st)
    rc = lib().oracle_blend_stitch(ptrs, N, C, n_t, n_h, n_w,
                                   _i64(list(ext_t) + list(ext_h) + list(ext_w)),
                                   _i64(blend), _i64(row_limit), DTYPE_CODE[dtype], _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_blend_stitch rejected the geometry (rc={rc})")
    return out


def blend_workload(w, tiles):
    """``blend_stitch`` for a ``workloads.BlendWorkload``."""
    return blend_stitch(tiles, w.N, w.C, w.ext_t, w.ext_h, w.ext_w, w.blend, w.row_limit,
                        w.dtype, ndim=w.ndim)


def ramp_weight(p, origin, extent, k, n, margin, ramp) -> float:
    """Weight of tile k of n (origin, extent) at position p along one axis."""
    return float(lib().oracle_ramp_weight(p, origin, extent, k, n, margin, ramp))


def ramp_blend(tiles, lead_shape, origins_h, extents_h, origins_w, extents_w, margin, ramp,
               dtype, with_magnitude=False):
    """Normalised-ramp blend of wide tiles, in double.  ``tiles`` are
    storage-form arrays of shape lead_shape + (extent_h_i, extent_w_j) in raster
    order; ``margin`` and ``ramp`` are (H, W) pairs in positions.  Returns the
    float64 output of shape lead_shape + (L_h, L_w) (and the weighted sum of
    magnitudes when asked)."""
    n_h, n_w = len(origins_h), len(origins_w)
    assert len(tiles) == n_h * n_w
    st = NP_STORAGE[dtype]
    P = int(np.prod(lead_shape)) if len(lead_shape) else 1
    keep = [np.ascontiguousarray(t, dtype=st) for t in tiles]
    for k, t in enumerate(keep):
        i, j = divmod(k, n_w)
        assert t.size == P * extents_h[i] * extents_w[j], "tile size mismatch"
    LH = max(o + e for o, e in zip(origins_h, extents_h))
    LW = max(o + e for o, e in zip(origins_w, extents_w))
    ptrs = (ctypes.c_void_p * len(keep))(*[t.ctypes.data for t in keep])
    out = np.empty(tuple(lead_shape) + (LH, LW), dtype=np.float64)
    mag = np.empty_like(out) if with_magnitude else None
    rc = lib().oracle_ramp_blend(ptrs, P, n_h, n_w, _i64(origins_h), _i64(extents_h),
                                 _i64(origins_w), _i64(extents_w), LH, LW, int(margin[0]),
                                 int(ramp[0]), int(margin[1]), int(ramp[1]), DTYPE_CODE[dtype],
                                 _ptr(out), None if mag is None else _ptr(mag))
    if rc != 0:
        raise ValueError(f"oracle_ramp_blend rejected the layout (rc={rc})")
    return (out, mag) if with_magnitude else out


def groupnorm(x, groups, eps, gamma, beta, dtype):
    """Unsplit GroupNorm in double.  Returns (y float64, mean [N,G], var [N,G])."""
    st = NP_STORAGE[dtype]
    x = np.ascontiguousarray(x, dtype=st)
    N = x.shape[0]
    y = np.empty(x.shape, dtype=np.float64)
    mean = np.empty((N, groups), dtype=np.float64)
    var = np.empty((N, groups), dtype=np.float64)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=st)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=st)
    rc = lib().oracle_groupnorm(_ptr(x), x.ndim, _i64(x.shape), groups, float(eps),
                                None if g is None else _ptr(g), None if b is None else _ptr(b),
                                DTYPE_CODE[dtype], _ptr(y), _ptr(mean), _ptr(var))
    if rc != 0:
        raise ValueError("oracle_groupnorm: bad arguments")
    return y, mean, var


def patch_stats(x, groups, split_axis, n_patches, dtype):
    """Per-patch (count, mean, M2) in double, shape [N, G, P, 3]."""
    st = NP_STORAGE[dtype]
    x = np.ascontiguousarray(x, dtype=st)
    out = np.empty((x.shape[0], groups, n_patches, 3), dtype=np.float64)
    rc = lib().oracle_patch_stats(_ptr(x), x.ndim, _i64(x.shape), groups, split_axis,
                                  n_patches, DTYPE_CODE[dtype], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_patch_stats: bad arguments")
    return out


def chan_merge(stats):
    """Chan merge over the patch axis of [..., P, 3] statistics -> [..., 3]."""
    stats = np.ascontiguousarray(stats, dtype=np.float64)
    P = stats.shape[-2]
    rows = int(np.prod(stats.shape[:-2]))
    out = np.empty(stats.shape[:-2] + (3,), dtype=np.float64)
    lib().oracle_chan_merge(_ptr(stats), rows, P, _ptr(out))
    return out


def coefficients(e: int):
    """(w_a, w_b) float32 arrays of length e."""
    wa = np.empty(max(1, e), dtype=np.float32)
    wb = np.empty(max(1, e), dtype=np.float32)
    lib().oracle_blend_coefficients(e, _ptr(wa), _ptr(wb))
    return wa[:e], wb[:e]


def crossfade(a: float, b: float, wa: float, wb: float, dtype: str) -> float:
    return float(lib().oracle_crossfade(a, b, wa, wb, DTYPE_CODE[dtype]))


def to_f16_bits(v: float) -> int:
    return int(lib().oracle_f32_to_f16(v))


def to_bf16_bits(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(v))


def round_to_storage_bits(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """The oracle's own fp32 -> fp16/bf16 round-to-nearest-even, as uint16 bits."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_round_f32_array(_ptr(v), v.size, DTYPE_CODE[dtype], _ptr(out))
    return out


def widen_storage_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """The oracle's own fp16/bf16 -> fp32 widening."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().oracle_widen_array(_ptr(b), b.size, DTYPE_CODE[dtype], _ptr(out))
    return out
