"""CPU checks of the C ABI: the library loads, exports every function the header
declares, and rejects bad arguments and geometries on the host (before any
device work, so these run without a GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seam_blend.h")


@pytest.fixture(scope="module")
def sb():
    import seam_blending_patch_amd as m  # raises if the library is not built
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["vae_tile_blend_stitch", "vae_tile_blend_stitch_output_extents", "patch_groupnorm",
              "patch_groupnorm_workspace_bytes", "seamblend_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(sb):
    lib = ctypes.CDLL(sb.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_output_extents_for_the_benchmark_grids(sb):
    want = {1: (1, 112, 112), 2: (1, 1024, 1024), 3: (1, 2048, 2048), 4: (49, 480, 832),
            5: (1, 4096, 4096)}
    for k, c in workloads.CONFIGS.items():
        w = c.blend
        grid = (w.ndim, w.N, w.C) + w.grid
        ext = list(w.ext_t) + list(w.ext_h) + list(w.ext_w)
        assert sb.vae_tile_blend_stitch_output_extents(grid, ext, w.blend, w.row_limit) == want[k]


@pytest.mark.parametrize("grid,ext,E,R,code", [
    ((3, 1, 3, 1, 2, 2), [1, 64, 64, 64, 64], (0, 16, 16), (1, 48, 48), -1),    # bad ndim
    ((4, 1, 3, 2, 2, 2), [1, 1, 64, 64, 64, 64], (0, 16, 16), (1, 48, 48), -1), # n_t != 1 in 4-D
    ((4, 1, 3, 1, 2, 2), [2, 64, 64, 64, 64], (0, 16, 16), (1, 48, 48), -1),    # t_0 != 1 in 4-D
    ((4, 1, 3, 1, 0, 2), [1, 64, 64], (0, 16, 16), (1, 48, 48), -1),            # empty grid axis
    ((4, 1, 3, 1, 2, 2), [1, 64, 64, 64, 64], (0, -1, 16), (1, 48, 48), -1),    # negative E
    ((4, 1, 3, 1, 2, 2), [1, 64, 64, 64, 64], (0, 16, 16), (1, 0, 48), -1),     # R = 0
    ((4, 1, 3, 1, 2, 2), [1, 40, 64, 64, 64], (0, 16, 16), (1, 48, 48), -2),    # non-last < R
    ((4, 1, 3, 1, 3, 1), [1, 64, 20, 64, 64], (0, 16, 16), (1, 20, 48), -2),    # head meets tail
    ((4, 1, 3, 1, 65, 1), [1] + [8] * 65 + [8], (0, 0, 0), (1, 8, 8), -2),      # > 64 tiles per axis
])
def test_geometry_validation(sb, grid, ext, E, R, code):
    with pytest.raises(sb.SeamBlendError) as ei:
        sb.vae_tile_blend_stitch_output_extents(grid, ext, E, R)
    assert ei.value.code == code
    assert len(str(ei.value)) > 20


def test_blend_rejects_bad_pointers_and_dtype_before_any_launch(sb):
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.vae_tile_blend_stitch.restype = ctypes.c_int
    lib.seamblend_last_error.restype = ctypes.c_char_p
    i64 = lambda v: (ctypes.c_int64 * len(v))(*v)  # noqa: E731
    grid, ext, E, R = i64([4, 1, 3, 1, 2, 2]), i64([1, 64, 64, 64, 64]), i64([0, 16, 16]), i64([1, 48, 48])
    fake = (ctypes.c_void_p * 4)(0x1000, 0x100000, 0x200000, 0x300000)
    assert lib.vae_tile_blend_stitch(fake, grid, ext, E, R, 7, ctypes.c_void_p(0x900000), None) == -1
    assert b"dtype" in lib.seamblend_last_error()
    assert lib.vae_tile_blend_stitch(None, grid, ext, E, R, 1, ctypes.c_void_p(0x900000), None) == -1
    assert lib.vae_tile_blend_stitch(fake, grid, ext, E, R, 1, None, None) == -1
    nul = (ctypes.c_void_p * 4)(0x1000, 0, 0x200000, 0x300000)
    assert lib.vae_tile_blend_stitch(nul, grid, ext, E, R, 1, ctypes.c_void_p(0x900000), None) == -1
    # output overlapping a tile
    assert lib.vae_tile_blend_stitch(fake, grid, ext, E, R, 1, ctypes.c_void_p(0x100010), None) == -1
    assert b"overlap" in lib.seamblend_last_error()
    # misaligned fp32 tile
    mis = (ctypes.c_void_p * 4)(0x1002, 0x100000, 0x200000, 0x300000)
    assert lib.vae_tile_blend_stitch(mis, grid, ext, E, R, 0, ctypes.c_void_p(0x900000), None) == -1


def test_groupnorm_workspace_and_validation(sb):
    assert sb.patch_groupnorm_workspace_bytes((1, 512, 256, 256), 32, 2, 4) > 0
    # the workspace does not depend on dtype: one size serves all
    a = sb.patch_groupnorm_workspace_bytes((2, 256, 512, 512), 32, 3, 8)
    assert a == 2 * 32 * 8 * 8 * 16  # (n, g, patch, 8 chunks) partials of 16 bytes
    for shape, G, axis, P in [((1, 30, 8, 8), 4, 2, 2),   # C % G
                              ((1, 32, 8, 8), 4, 1, 2),   # axis not spatial
                              ((1, 32, 8, 8), 4, 4, 2),   # axis out of range
                              ((1, 32, 8, 8), 4, 2, 0),   # no patches
                              ((1, 32, 8, 8), 4, 2, 65),  # too many patches
                              ((1, 32), 4, 2, 1),         # rank
                              ((1, 2, 1 << 15, 1 << 15), 1, 2, 1),  # a group of 2^31 elements
                              ((1 << 20, 4096, 1, 1), 4096, 2, 1)]:  # N*C of 2^32 planes
        with pytest.raises(sb.SeamBlendError):
            sb.patch_groupnorm_workspace_bytes(shape, G, axis, P)
    # more (n, c) planes than one launch's grid holds in y: accepted (pass 2
    # takes several launches); one chunk per patch at 8 elements per chunk
    assert sb.patch_groupnorm_workspace_bytes((2, 65536, 4, 4), 256, 2, 2) == 2 * 256 * 2 * 16
    # a group just below 2^31 elements is accepted
    assert sb.patch_groupnorm_workspace_bytes((1, 2, (1 << 15) - 1, 1 << 15), 1, 2, 1) > 0


def test_groupnorm_rejects_small_workspace_and_bad_args_on_host(sb):
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.patch_groupnorm.restype = ctypes.c_int
    lib.patch_groupnorm.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    shape = (ctypes.c_int64 * 4)(1, 8, 16, 16)
    X, Y, W = 0x10000, 0x20000, 0x30000
    assert lib.patch_groupnorm(X, 4, shape, 4, 2, 2, 1e-6, None, None, 0, Y, W, 4, None, None) == -3
    assert lib.patch_groupnorm(X, 4, shape, 4, 2, 2, -1.0, None, None, 0, Y, W, 4096, None, None) == -1
    assert lib.patch_groupnorm(X, 4, shape, 4, 2, 2, 1e-6, None, None, 9, Y, W, 4096, None, None) == -1
    assert lib.patch_groupnorm(None, 4, shape, 4, 2, 2, 1e-6, None, None, 0, Y, W, 4096, None, None) == -1
    assert lib.patch_groupnorm(X, 4, shape, 4, 2, 2, 1e-6, None, None, 0, X + 64, W, 4096, None,
                               None) == -1  # partial overlap of out and x
    # empty tensors are a no-op that needs no workspace
    empty = (ctypes.c_int64 * 4)(0, 8, 16, 16)
    assert lib.patch_groupnorm(X, 4, empty, 4, 2, 2, 1e-6, None, None, 0, Y, None, 0, None, None) == 0


def _ramp_call(lib, grid, origins, extents, margin=(0, 4, 4), ramp=(0, 8, 8), dtype=2, out=0x900000,
               ptrs=None):
    i64 = lambda v: (ctypes.c_int64 * len(v))(*v)  # noqa: E731
    n = grid[4] * grid[5]
    fake = ptrs if ptrs is not None else (ctypes.c_void_p * max(1, n))(*[0x100000 * (k + 1) for k in range(n)])
    return lib.vae_tile_ramp_blend(fake, i64(grid), i64(origins), i64(extents), i64(margin), i64(ramp),
                                   dtype, ctypes.c_void_p(out) if out else None, None)


@pytest.mark.parametrize("grid,origins,extents,margin,ramp,dtype,code,needle", [
    ((3, 1, 3, 1, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32], (0, 4, 4), (0, 8, 8), 2, -1, "ndim"),
    ((4, 1, 3, 2, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32], (0, 4, 4), (0, 8, 8), 2, -1, "frames"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32], (0, -1, 4), (0, 8, 8), 2, -1, "margin"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32], (0, 4, 4), (0, 8, 0), 2, -1, "ramp"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 0, 0], [1, 32, 32, 32], (0, 4, 4), (0, 8, 8), 2, -2, "increase"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 4, 16], [1, 32, 32, 32], (0, 4, 4), (0, 8, 8), 2, -2, "start at 0"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 0, 16], [1, 32, 40, 8], (0, 4, 4), (0, 8, 8), 2, -2, "ends past"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 0, 23], [1, 32, 32, 32], (0, 4, 4), (0, 8, 8), 2, -2, "no tile has weight"),
    ((4, 1, 3, 1, 1, 5), [0, 0, 0, 2, 4, 6, 8], [1, 32] + [32] * 5, (0, 0, 0), (0, 8, 8), 2, -2, "at most"),
    ((4, 1, 3, 1, 1, 49), [0, 0] + [k for k in range(49)], [1, 32] + [32] * 49, (0, 0, 0), (0, 8, 8), 2,
     -1, "tiles per axis"),
    ((4, 1, 3, 1, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32], (0, 4, 4), (0, 8, 8), 7, -1, "dtype"),
])
def test_ramp_rejects_bad_layouts_on_host(sb, grid, origins, extents, margin, ramp, dtype, code, needle):
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.vae_tile_ramp_blend.restype = ctypes.c_int
    lib.seamblend_last_error.restype = ctypes.c_char_p
    assert _ramp_call(lib, grid, origins, extents, margin, ramp, dtype) == code
    assert needle.encode() in lib.seamblend_last_error()


def test_ramp_rejects_bad_pointers_on_host(sb):
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.vae_tile_ramp_blend.restype = ctypes.c_int
    lib.seamblend_last_error.restype = ctypes.c_char_p
    g, o, e = (4, 1, 3, 1, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32]
    assert _ramp_call(lib, g, o, e, out=0) == -1
    nul = (ctypes.c_void_p * 2)(0x100000, 0)
    assert _ramp_call(lib, g, o, e, ptrs=nul) == -1
    mis = (ctypes.c_void_p * 2)(0x100001, 0x200000)
    assert _ramp_call(lib, g, o, e, ptrs=mis) == -1
    assert _ramp_call(lib, g, o, e, out=0x100010) == -1
    assert b"overlaps" in lib.seamblend_last_error()
    # an empty batch is a no-op before any pointer is looked at
    assert _ramp_call(lib, (4, 0, 3, 1, 1, 2), o, e, out=0, ptrs=(ctypes.c_void_p * 2)(0, 0)) == 0


def test_sizes_beyond_the_index_range_are_rejected_on_host(sb):
    # N * C at 2^31 or more, or an output beyond 2^50 elements: rejected
    # before any pointer is used
    with pytest.raises(sb.SeamBlendError) as ei:
        sb.vae_tile_blend_stitch_output_extents((4, 1 << 31, 1, 1, 2, 2), [1, 64, 64, 64, 64], (0, 16, 16),
                                                (1, 48, 48))
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.vae_tile_blend_stitch.restype = ctypes.c_int
    i64 = lambda v: (ctypes.c_int64 * len(v))(*v)  # noqa: E731
    fake = (ctypes.c_void_p * 4)(0x1000, 0x100000, 0x200000, 0x300000)
    assert lib.vae_tile_blend_stitch(fake, i64([4, 1 << 31, 3, 1, 2, 2]), i64([1, 64, 64, 64, 64]),
                                     i64([0, 16, 16]), i64([1, 48, 48]), 1, ctypes.c_void_p(0x900000),
                                     None) == -2
    assert lib.vae_tile_blend_stitch(fake, i64([4, 1 << 20, 1 << 10, 1, 2, 2]),
                                     i64([1, 1 << 20, 1 << 20, 64, 64]), i64([0, 16, 16]),
                                     i64([1, 1 << 20, 48]), 1, ctypes.c_void_p(0x900000), None) == -2
    lib.vae_tile_ramp_blend.restype = ctypes.c_int
    assert _ramp_call(lib, (5, 1 << 16, 1 << 16, 1, 1, 2), [0, 0, 0, 16], [1, 32, 32, 32]) == -2
    # one temporal tile of 2^25 frames in the narrow-seam layout (two 8-wide
    # tile columns, 4-column seam): its grid's x extent takes the window's
    # frames, and 2^25 exceed the 2^24 - 1 blocks it allows, refused before any
    # launch (the segment layout takes any frame count, in ranges)
    two = (ctypes.c_void_p * 2)(0x1000, 1 << 40)
    lib.seamblend_last_error.restype = ctypes.c_char_p
    assert lib.vae_tile_blend_stitch(two, i64([5, 1, 1, 1, 1, 2]), i64([1 << 25, 1, 8, 8]), i64([0, 0, 4]),
                                     i64([1, 1, 8]), 0, ctypes.c_void_p(1 << 41), None) == -2
    assert b"frames exceeds" in lib.seamblend_last_error()


def test_too_wide_tile_grid_is_refused_before_any_launch(sb):
    # 64 tile columns, 2 tile rows, 2 temporal tiles: the first launch windows
    # fit the 192-entry pointer table, the window of tile row 1 in temporal
    # tile 1 (with the row above and the chunk before: 4 x 64 pointers) does
    # not.  Every window is planned first, so the call fails with a geometry
    # error before it launches anything (a launch here, with no GPU, would
    # report a launch error instead).
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.vae_tile_blend_stitch.restype = ctypes.c_int
    lib.seamblend_last_error.restype = ctypes.c_char_p
    i64 = lambda v: (ctypes.c_int64 * len(v))(*v)  # noqa: E731
    n = 2 * 2 * 64
    fake = (ctypes.c_void_p * n)(*[(k + 1) << 16 for k in range(n)])
    rc = lib.vae_tile_blend_stitch(fake, i64([5, 1, 1, 2, 2, 64]), i64([4, 4, 8, 8] + [8] * 64),
                                   i64([0, 0, 0]), i64([4, 8, 8]), 0, ctypes.c_void_p(1 << 40), None)
    assert rc == -2
    assert b"too wide" in lib.seamblend_last_error()


def test_row_limit_and_blend_extent_beyond_32_bits(sb):
    # a row limit above 2^30 is rejected (it would not fit the kernel's 32-bit
    # index arithmetic); a huge blend extent is the same as one clamped to the
    # tile extents
    with pytest.raises(sb.SeamBlendError) as ei:
        sb.vae_tile_blend_stitch_output_extents((4, 1, 3, 1, 1, 1), [1, 64, 64], (0, 16, 16),
                                                (1, 1 << 32, 48))
    assert ei.value.code == -1
    assert sb.vae_tile_blend_stitch_output_extents((4, 1, 3, 1, 2, 2), [1, 64, 64, 64, 64],
                                                   (0, 1 << 40, 1 << 40), (1, 48, 48)) == (1, 112, 112)


def test_ramp_output_beyond_2_50_elements_is_rejected(sb):
    lib = ctypes.CDLL(sb.LIB_PATH)
    lib.vae_tile_ramp_blend.restype = ctypes.c_int
    big = (1 << 19) + 16
    assert _ramp_call(lib, (4, 1 << 15, 1 << 15, 1, 1, 2), [0, 0, 0, 16], [1, big, 32, 32]) == -2
