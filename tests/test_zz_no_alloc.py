"""The allocation-free GroupNorm entry point (statistics in the library's
static per-GPU scratch) against patch_groupnorm with a caller workspace, both
called through the C ABI: bit-identical outputs and per-patch statistics on
two calls in a row, the second on a smaller problem, and within the oracle's
tolerance; a problem whose statistics exceed the static scratch is refused on
the host."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import compare
import oracle
import workloads
from gpu_util import as_f64, from_dev, to_dev

pytestmark = pytest.mark.gpu

DT = {"fp32": 0, "fp16": 1, "bf16": 2}


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import seam_blending_patch_amd as sb
    L = ctypes.CDLL(sb.LIB_PATH)
    i64p = ctypes.POINTER(ctypes.c_int64)
    common = [ctypes.c_void_p, ctypes.c_int, i64p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
              ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.patch_groupnorm.argtypes = common + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.patch_groupnorm.restype = ctypes.c_int
    L.patch_groupnorm_noalloc.argtypes = common + [ctypes.c_void_p, ctypes.c_void_p]
    L.patch_groupnorm_noalloc.restype = ctypes.c_int
    L.patch_groupnorm_workspace_bytes.argtypes = [ctypes.c_int, i64p, ctypes.c_int64, ctypes.c_int,
                                                  ctypes.c_int64]
    L.patch_groupnorm_workspace_bytes.restype = ctypes.c_size_t
    L.seamblend_last_error.restype = ctypes.c_char_p
    return L


def _shape(gw):
    return (ctypes.c_int64 * len(gw.shape))(*gw.shape)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _both(lib, gw, x, g, b):
    xd, gd, bd = to_dev(x, gw.dtype), to_dev(g, gw.dtype), to_dev(b, gw.dtype)
    n_st = gw.shape[0] * gw.groups * gw.n_patches * 3
    y_ws, y_na = torch.full_like(xd, float("nan")), torch.full_like(xd, float("nan"))
    st_ws = torch.full((n_st,), float("nan"), device="cuda")
    st_na = torch.full((n_st,), float("nan"), device="cuda")
    need = lib.patch_groupnorm_workspace_bytes(len(gw.shape), _shape(gw), gw.groups, gw.split_axis,
                                               gw.n_patches)
    assert 0 < need <= 1 << 20
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = lib.patch_groupnorm(_ptr(xd), len(gw.shape), _shape(gw), gw.groups, gw.split_axis, gw.n_patches,
                             gw.eps, _ptr(gd), _ptr(bd), DT[gw.dtype], _ptr(y_ws), _ptr(ws), need,
                             _ptr(st_ws), _stream())
    assert rc == 0, lib.seamblend_last_error()
    rc = lib.patch_groupnorm_noalloc(_ptr(xd), len(gw.shape), _shape(gw), gw.groups, gw.split_axis,
                                     gw.n_patches, gw.eps, _ptr(gd), _ptr(bd), DT[gw.dtype], _ptr(y_na),
                                     _ptr(st_na), _stream())
    assert rc == 0, lib.seamblend_last_error()
    torch.cuda.synchronize()
    return y_ws, y_na, st_ws, st_na


def test_noalloc_equals_the_workspace_entry_point_on_two_calls(lib):
    # first the video-decoder activation (bf16, 4 patches along H), then the
    # smaller 32x32 fp32 one: the second call reuses the scratch the first left
    for cfg in (4, 1):
        gw, (x, g, b) = workloads.draw_config_groupnorm(cfg)
        print(f"[noalloc] config {cfg} {gw.shape} {gw.dtype}", file=sys.stderr, flush=True)
        y_ws, y_na, st_ws, st_na = _both(lib, gw, x, g, b)
        bits = torch.int32 if gw.dtype == "fp32" else torch.int16
        assert torch.equal(y_na.view(bits), y_ws.view(bits)), f"config {cfg}: outputs differ"
        assert torch.equal(st_na.view(torch.int32), st_ws.view(torch.int32)), f"config {cfg}: patch stats"
        ref, _, _ = oracle.groupnorm(x, gw.groups, gw.eps, g, b, gw.dtype)
        ok, rep = compare.groupnorm_check(as_f64(from_dev(y_na, gw.dtype), gw.dtype), ref, gw.dtype)
        assert ok, f"config {cfg}: {rep}"


def test_noalloc_refuses_statistics_beyond_the_static_scratch(lib):
    # 64 x 32 groups x 64 patches, one chunk each: 2 MiB of partials; refused
    # on the host before anything is enqueued (the pointers are never used)
    shape = (ctypes.c_int64 * 4)(64, 512, 64, 64)
    need = lib.patch_groupnorm_workspace_bytes(4, shape, 32, 2, 64)
    assert need > 1 << 20
    rc = lib.patch_groupnorm_noalloc(ctypes.c_void_p(0x10000), 4, shape, 32, 2, 64, 1e-6, None, None, 2,
                                     ctypes.c_void_p(0x20000), None, None)
    assert rc == -3
    assert b"static" in lib.seamblend_last_error()
