"""Independent brute-force models used to pin the C oracle (test-only).

Two blend models, both written separately from ``oracle/oracle.c`` and from the
HIP kernels:

* ``literal_torch`` -- the literal in-place raster algorithm, one vectorised
  torch CPU expression per seam (the shape of the prior-art broadcast), with
  rounding done by torch's own dtype conversions.
* ``closed_form_numpy`` -- a per-output-element closed form (derived, not
  stated on the pages): every output element depends on at most 4 tiles in
  2-D (8 in 5-D) given the tile geometry preconditions.  numpy float32 ops do
  the fp32 arithmetic; numpy float16 / torch bfloat16 conversions do RN_T.

Agreement of three implementations that share no code (C literal, torch
literal, numpy closed form) is one of the pins of the oracle; the others are
in tests/test_oracle_blend.py.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


# ---------------------------------------------------------------------------
# storage helpers (library conversions only)
# ---------------------------------------------------------------------------
def storage_to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(arr, dtype=np.float32)
    if dtype == "fp16":
        return np.asarray(arr, dtype=np.float16).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).float().numpy()


def f32_to_storage(v: np.ndarray, dtype: str) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    if dtype == "fp32":
        return v
    if dtype == "fp16":
        return v.astype(np.float16)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rn(v: np.ndarray, dtype: str) -> np.ndarray:
    """RN_T through library conversions, widened back to float32."""
    return storage_to_f32(f32_to_storage(v, dtype), dtype)


def to_torch(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr))


def from_torch(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def coeff_f32(e: int):
    """(w_a, w_b) as float32 from Python double division (the definition)."""
    wb = np.array([k / e for k in range(e)], dtype=np.float64).astype(np.float32)
    wa = np.array([1.0 - k / e for k in range(e)], dtype=np.float64).astype(np.float32)
    return wa, wb


# ---------------------------------------------------------------------------
# geometry (restated independently of the oracle and the library)
# ---------------------------------------------------------------------------
def _axis(exts, E, R):
    n = len(exts)
    e = [0] + [min(E, exts[k - 1], exts[k]) for k in range(1, n)]
    crop = [R if k < n - 1 else exts[-1] for k in range(n)]
    return e, crop, (n - 1) * R + exts[-1]


def _tiles5(w, tiles):
    """storage tiles -> float32 arrays of shape [N,C,t,h,w] indexed [tau][i][j]."""
    nt, nh, nw = w.grid
    out = [[[None] * nw for _ in range(nh)] for _ in range(nt)]
    k = 0
    for tau in range(nt):
        for i in range(nh):
            for j in range(nw):
                a = storage_to_f32(tiles[k], w.dtype)
                out[tau][i][j] = a.reshape(w.N, w.C, w.ext_t[tau], w.ext_h[i], w.ext_w[j])
                k += 1
    return out


# ---------------------------------------------------------------------------
# literal algorithm with torch CPU ops
# ---------------------------------------------------------------------------
def literal_torch(w, tiles, in_place: bool = True, temporal_first: bool = False):
    """Literal blend+crop+stitch.  ``in_place=False`` (reading the original,
    unblended neighbours) and ``temporal_first=True`` (blend_t before the
    spatial pass) are the wrong variants, used to show the pins can tell them
    apart."""
    dt = TORCH_DT[w.dtype]
    nt, nh, nw = w.grid
    Et, Eh, Ew = w.blend
    Rt, Rh, Rw = w.row_limit
    T = [[[None] * nw for _ in range(nh)] for _ in range(nt)]
    k = 0
    for tau in range(nt):
        for i in range(nh):
            for j in range(nw):
                t = to_torch(tiles[k], w.dtype).reshape(w.N, w.C, w.ext_t[tau], w.ext_h[i], w.ext_w[j])
                T[tau][i][j] = t.clone()
                k += 1

    def crossfade(a, b, dim, e):
        # coefficient vector from float64 division, rounded once to float32
        kk = torch.arange(e, dtype=torch.float64)
        wb = (kk / e).to(torch.float32)
        wa = (1.0 - kk / e).to(torch.float32)
        shape = [1] * a.dim()
        shape[dim] = e
        wa, wb = wa.reshape(shape), wb.reshape(shape)
        pa = (a.to(torch.float32) * wa).to(dt)
        pb = (b.to(torch.float32) * wb).to(dt)
        return (pa.to(torch.float32) + pb.to(torch.float32)).to(dt)

    def blend(a, b, dim, E):
        e = min(E, a.shape[dim], b.shape[dim])
        if e <= 0:
            return b
        tail = a.narrow(dim, a.shape[dim] - e, e)
        head = b.narrow(dim, 0, e)
        b = b.clone()
        b.narrow(dim, 0, e).copy_(crossfade(tail, head, dim, e))
        return b

    def spatial(tau_tiles):
        src = [[tau_tiles[i][j] for j in range(nw)] for i in range(nh)]
        B = [[tau_tiles[i][j].clone() for j in range(nw)] for i in range(nh)]
        for i in range(nh):
            for j in range(nw):
                if i > 0:
                    a = B[i - 1][j] if in_place else src[i - 1][j]
                    B[i][j] = blend(a, B[i][j], 3, Eh)
                if j > 0:
                    a = B[i][j - 1] if in_place else src[i][j - 1]
                    B[i][j] = blend(a, B[i][j], 4, Ew)
        rows = []
        for i in range(nh):
            ch = Rh if i < nh - 1 else B[i][0].shape[3]
            row = [B[i][j][:, :, :, :ch, : (Rw if j < nw - 1 else B[i][j].shape[4])] for j in range(nw)]
            rows.append(torch.cat(row, dim=4))
        return torch.cat(rows, dim=3)

    if temporal_first:
        # wrong order: temporal blend of each spatial tile column first
        for i in range(nh):
            for j in range(nw):
                for tau in range(1, nt):
                    T[tau][i][j] = blend(T[tau - 1][i][j], T[tau][i][j], 2, Et)
        chunks = [spatial(T[tau]) for tau in range(nt)]
    else:
        chunks = [spatial(T[tau]) for tau in range(nt)]
        for tau in range(1, nt):
            chunks[tau] = blend(chunks[tau - 1], chunks[tau], 2, Et)
    parts = [chunks[tau][:, :, : (Rt if tau < nt - 1 else chunks[tau].shape[2])] for tau in range(nt)]
    out = torch.cat(parts, dim=2)
    if w.ndim == 4:
        out = out[:, :, 0]
    return from_torch(out, w.dtype)


# ---------------------------------------------------------------------------
# closed form, per output cell, numpy float32
# ---------------------------------------------------------------------------
def closed_form_numpy(w, tiles):
    dt = w.dtype
    D = _tiles5(w, tiles)
    nt, nh, nw = w.grid
    et, ct, LT = _axis(w.ext_t, w.blend[0], w.row_limit[0])
    eh, ch, LH = _axis(w.ext_h, w.blend[1], w.row_limit[1])
    ew, cw, LW = _axis(w.ext_w, w.blend[2], w.row_limit[2])
    Rt, Rh, Rw = w.row_limit

    def beta(a, b, wa, wb):
        pa = rn(a * wa, dt)
        pb = rn(b * wb, dt)
        return rn(pa + pb, dt)

    def spatial(tau, frames, i, j):
        """S_tau over the crop of cell (i, j) at the given frames."""
        h_i, w_j = ch[i], cw[j]
        s = D[tau][i][j][:, :, frames, :h_i, :w_j].copy()
        E_h, E_w = eh[i], ew[j]
        # seam rows / columns that survive the crop
        nh_, nw_ = min(E_h, h_i), min(E_w, w_j)
        u = w.ext_h[i - 1] - E_h if E_h > 0 else 0
        l = w.ext_w[j - 1] - E_w if E_w > 0 else 0
        if E_h > 0:
            wa_h, wb_h = (c[:nh_] for c in coeff_f32(E_h))
        if E_w > 0:
            wa_w, wb_w = (c[:nw_] for c in coeff_f32(E_w))
        if E_h > 0:
            U = D[tau][i - 1][j][:, :, frames, u:u + nh_, :w_j].copy()
            if E_w > 0:
                Cn = D[tau][i - 1][j - 1][:, :, frames, u:u + nh_, l:l + nw_]
                U[..., :nw_] = beta(Cn, U[..., :nw_], wa_w, wb_w)
            s_old = s.copy()
            s[..., :nh_, :] = beta(U, s_old[..., :nh_, :], wa_h[:, None], wb_h[:, None])
        if E_w > 0:
            Lf = D[tau][i][j - 1][:, :, frames, :h_i, l:l + nw_].copy()
            if E_h > 0:
                Cn = D[tau][i - 1][j - 1][:, :, frames, u:u + nh_, l:l + nw_]
                Lf[..., :nh_, :] = beta(Cn, Lf[..., :nh_, :], wa_h[:, None], wb_h[:, None])
            s[..., :nw_] = beta(Lf, s[..., :nw_], wa_w, wb_w)
        return s

    out = np.zeros((w.N, w.C, LT, LH, LW), dtype=np.float32)
    for tau in range(nt):
        f_all = np.arange(ct[tau])
        for i in range(nh):
            for j in range(nw):
                S = spatial(tau, f_all, i, j)
                E_t = et[tau]
                if E_t > 0:
                    nf = min(E_t, ct[tau])
                    p = w.ext_t[tau - 1] - E_t
                    wa_t, wb_t = (c[:nf] for c in coeff_f32(E_t))
                    Sp = spatial(tau - 1, np.arange(p, p + nf), i, j)
                    S[:, :, :nf] = beta(Sp, S[:, :, :nf], wa_t[:, None, None], wb_t[:, None, None])
                out[:, :, tau * Rt: tau * Rt + ct[tau], i * Rh: i * Rh + ch[i],
                    j * Rw: j * Rw + cw[j]] = S
    if w.ndim == 4:
        out = out[:, :, 0]
    return f32_to_storage(out, dt)


# ---------------------------------------------------------------------------
# exact-arithmetic helpers
# ---------------------------------------------------------------------------
def correctly_rounded_f32(x: Fraction) -> np.float32:
    """The binary32 value nearest to the rational x (ties to even), found by
    comparing the neighbours of a candidate exactly."""
    c = np.float32(float(x))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - x)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best = (d, np.float32(cand))
    return best[1]
