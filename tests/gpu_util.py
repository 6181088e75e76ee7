"""Helpers for the GPU parity tests: move storage-form numpy arrays to and from
the device without any arithmetic."""
from __future__ import annotations

import numpy as np
import torch

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def tile_grid(w, tiles_np, device="cuda"):
    """Storage tiles (raster order) -> nested device tensors for the binding."""
    nt, nh, nw = w.grid
    dev = [to_dev(t, w.dtype, device) for t in tiles_np]
    k = 0
    grid = []
    for tau in range(nt):
        plane = []
        for i in range(nh):
            row = []
            for j in range(nw):
                row.append(dev[k].reshape(w.tile_shape(tau, i, j)))
                k += 1
            plane.append(row)
        grid.append(plane)
    return grid[0] if w.ndim == 4 else grid


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)
