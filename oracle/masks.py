"""Fixed block masks as per-query-tile ascending key-tile lists.

Follows:
  * FPSAttention summary page, "Approach" and the ablation table: tile-wise
    structured sparse attention with a 3D sliding window over tiles, the
    window size being a tunable (e.g. (6,6,6) vs (6,6,1));
  * OSP-Next model card, "Model Summary" and the wiki TL;DR: Skiparse-2D is a
    fixed strided pattern along H and W, mixed with full-attention layers.

Readings:
  * window: key tile kept iff |delta| <= r per axis in tile coordinates,
    clipped at the grid edge (no wrap, no shifting the window inward); a key
    tile is kept even if it is partly padding;
  * Skiparse-2D: a query attends exactly the keys of its own residue group,
    so its key tiles are all tiles of its group;
  * any negative radius means dense: every tile is listed.
"""
from __future__ import annotations

from typing import List

from .layout import Layout, tile_coords, tile_group


def window_lists(lay: Layout, rt: int, rh: int, rw: int) -> List[List[int]]:
    """Per query tile, the ascending key tiles inside the +-(rt, rh, rw) window."""
    if rt < 0 or rh < 0 or rw < 0:
        return dense_lists(lay)
    if lay.kind == "skiparse2d":
        return skiparse_lists(lay)
    lists = []
    for qt in range(lay.n_tiles):
        a, b, c = tile_coords(lay, qt)
        row = []
        for kt in range(lay.n_tiles):
            a2, b2, c2 = tile_coords(lay, kt)
            if abs(a - a2) <= rt and abs(b - b2) <= rh and abs(c - c2) <= rw:
                row.append(kt)
        lists.append(row)
    return lists


def skiparse_lists(lay: Layout) -> List[List[int]]:
    """Per query tile, every key tile of the same residue group."""
    lists = []
    for qt in range(lay.n_tiles):
        g = tile_group(lay, qt)
        lists.append([kt for kt in range(lay.n_tiles) if tile_group(lay, kt) == g])
    return lists


def dense_lists(lay: Layout) -> List[List[int]]:
    return [list(range(lay.n_tiles)) for _ in range(lay.n_tiles)]


def group_range(X: int, extent: int, n_groups: int):
    """Groups X - (e-1)//2 .. X - (e-1)//2 + e - 1, clipped to 0 .. n_groups-1 (inclusive)."""
    lo = X - (extent - 1) // 2
    return max(lo, 0), min(lo + extent - 1, n_groups - 1)


def window_lists_grouped(lay: Layout, group, extent) -> List[List[int]]:
    """Per query tile, the ascending key tiles of every tile group inside the
    window of its own group (3D tiles only).

    FPSAttention summary, Approach and ablation table: quantisation and
    sparsity share one tile granularity, which changes across denoising steps;
    hardware-friendly (6,8,8) tiles and asymmetric windows such as (6,6,1).
    Readings: a big tile is a group of group = (gt, gh, gw) consecutive tiles
    of the layout's tile grid (e.g. (6,1,1) groups of (1,8,8) tiles form
    (6,8,8) tiles, the last group along an axis possibly shorter); a window
    extent e counts groups along its axis, covering X - (e-1)//2 ..
    X - (e-1)//2 + e - 1 around the query's group X (the extra group of an
    even extent on the high side), clipped at the grid edge without shifting.
    """
    assert lay.kind == "tile3d"
    nt, nh, nw = lay.tile_grid
    gt, gh, gw = group
    ng = (-(-nt // gt), -(-nh // gh), -(-nw // gw))
    lists = []
    for qt in range(lay.n_tiles):
        a, b, c = tile_coords(lay, qt)
        rng = [group_range(x, e, n) for x, e, n in zip((a // gt, b // gh, c // gw), extent, ng)]
        row = []
        for kt in range(lay.n_tiles):
            a2, b2, c2 = tile_coords(lay, kt)
            if all(lo <= x <= hi for (lo, hi), x in zip(rng, (a2 // gt, b2 // gh, c2 // gw))):
                row.append(kt)
        lists.append(row)
    return lists
