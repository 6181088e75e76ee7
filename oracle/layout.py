"""CPU oracle for tile layouts along one axis of a tiled decode.

TEST INFRASTRUCTURE ONLY: imported by tests/ and nothing else; it shares no
code with the library's planner.  Every rule is written as a search over the
candidate layouts, checked by building the tiles and measuring them, rather
than as a closed form, so that it can be compared with the library's closed
forms.

Rules (unsloth Studio PR "size seam-free VAE tiles from measured peaks (no
slower than stock, no low-VRAM OOM)", sections "Problem" and "Change" and the
commit messages it carries):

* ``stock``: the diffusers loop -- a tile of ``T`` at every multiple of the
  stride ``S`` below the canvas, the last ones cut short by the edge.
* ``edge_aligned``: the wide tiles of the Qwen-Image-2.1 commit -- side ``t``,
  neighbours overlapping by at least ``ov``, spread evenly so the last tile
  ends at the edge at full size; a canvas within one tile is one tile.
* ``fewest_calls``: the sliver rule for a VAE whose stock tile is the floor
  tile -- among layouts whose decoded latents along the axis do not exceed the
  stock loop's, the fewest tiles, then the widest (at most ``M``).  The pages'
  test list allows the bound "up to rounding"; read as: when no whole-latent
  side of n tiles fits the budget but the exact fractional covering side does
  (L + (n - 1) ov <= budget), the covering side rounded up is taken.
* ``smallest_side``: the fewest tiles of side at most ``M`` that cover with the
  overlap, then the smallest such side (the earlier rule, kept for the
  32-latent-floor VAEs).
* ``auto``: the rule of the "every image VAE" commit -- keep the stock tiles
  when every tile is at least ``floor_tile`` and every overlap at least
  ``floor_overlap``; otherwise edge-aligned tiles of ``max(floor_tile, T)``
  with overlap ``max(floor_overlap, T - S)``.

"Spread evenly" is read as origin_k = floor(k (L - t) / (n - 1)): the first
tile at 0, the last at L - t, the gaps differing by at most one latent.

Pins: tests/golden/layout_pages.json holds the layouts the pages print, and
tests/test_layout.py checks the properties the pages' test list states.
"""
from __future__ import annotations

from typing import List, Tuple

Tiles = List[Tuple[int, int]]  # (origin, extent)


def stock(L: int, T: int, S: int) -> Tiles:
    if S > T:
        raise ValueError("a stride above the tile leaves gaps")
    tiles = []
    o = 0
    while o < L:
        tiles.append((o, min(T, L - o)))
        o += S
    return tiles


def spread(L: int, t: int, n: int) -> Tiles:
    if n == 1:
        return [(0, t)]
    return [(k * (L - t) // (n - 1), t) for k in range(n)]


def overlaps(tiles: Tiles) -> List[int]:
    return [a_o + a_e - b_o for (a_o, a_e), (b_o, _) in zip(tiles, tiles[1:])]


def covers(L: int, tiles: Tiles, ov: int) -> bool:
    """Tiles inside [0, L), the first at 0, the last ending at L, origins
    increasing, and every neighbour overlap at least ``ov``."""
    if not tiles or tiles[0][0] != 0:
        return False
    if any(o < 0 or e < 1 or o + e > L for o, e in tiles):
        return False
    if max(o + e for o, e in tiles) != L:
        return False
    if any(b[0] <= a[0] for a, b in zip(tiles, tiles[1:])):
        return False
    return all(x >= ov for x in overlaps(tiles))


def edge_aligned(L: int, t: int, ov: int) -> Tiles:
    if L <= t:
        return [(0, L)]
    for n in range(2, L + 1):
        if covers(L, spread(L, t, n), ov):
            return spread(L, t, n)
    raise ValueError("no tiles of this side cover with this overlap")


def decoded(tiles: Tiles) -> int:
    return sum(e for _, e in tiles)


def fewest_calls(L: int, T: int, S: int, ov: int, M: int) -> Tiles:
    budget = decoded(stock(L, T, S))
    if L <= M:
        return [(0, L)]  # one call over the whole canvas; the stock loop decodes >= L
    for n in range(2, L + 1):
        if L + (n - 1) * ov > budget:
            break  # n tiles overlapping by >= ov decode at least L + (n - 1) ov latents
        top = min(M, L)
        if not covers(L, spread(L, top, n), ov):
            continue  # a narrower side covers less: no n-tile layout
        t = min(top, budget // n)  # the widest side within the budget
        if t >= 1 and covers(L, spread(L, t, n), ov):
            return spread(L, t, n)
        # "no more latents up to rounding": n tiles overlapping by exactly ov
        # decode L + (n - 1) ov latents at the fractional side that just
        # covers; that fits (checked above), so the side rounded up to whole
        # latents is taken
        t = 1
        while not covers(L, spread(L, t, n), ov):
            t += 1
        return spread(L, t, n)
    raise ValueError("no layout decodes within the stock budget")


def smallest_side(L: int, ov: int, M: int) -> Tiles:
    if L <= M:
        return [(0, L)]
    for n in range(2, L + 1):
        if not covers(L, spread(L, M, n), ov):
            continue  # a narrower side covers less
        for t in range(1, M + 1):  # smallest first
            if covers(L, spread(L, t, n), ov):
                return spread(L, t, n)
    raise ValueError("no side of at most M covers with this overlap")


def auto(L: int, T: int, S: int, floor_tile: int, floor_overlap: int) -> Tiles:
    st = stock(L, T, S)
    if len(st) == 1 or (all(e >= floor_tile for _, e in st)
                        and all(x >= floor_overlap for x in overlaps(st))):
        return st
    return edge_aligned(L, max(floor_tile, T), max(floor_overlap, T - S))


def layout(L: int, rule: str, params) -> Tiles:
    p = list(params)
    if rule == "stock":
        return stock(L, p[0], p[1])
    if rule == "edge_aligned":
        return edge_aligned(L, p[0], p[1])
    if rule == "fewest_calls":
        return fewest_calls(L, p[0], p[1], p[2], p[3])
    if rule == "smallest_side":
        return smallest_side(L, p[0], p[1])
    if rule == "auto":
        return auto(L, p[0], p[1], p[2], p[3])
    raise ValueError(rule)
