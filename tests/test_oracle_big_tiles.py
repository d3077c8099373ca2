"""Pins for the big-tile (grouped) windows and the grouped fp8 quantiser
(FPSAttention, Approach and ablation table: (6,8,8) tiles, windows such as
(6,6,1), quantisation on the same tiles as the sparsity)."""
import os

import numpy as np
import pytest

from oracle import fp8 as F
from oracle import layout as L
from oracle import masks as M
from oracle.layout import Layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "grouped_windows.txt")


def test_grouped_windows_golden():
    lay = Layout(T=5, H=2, W=6, heads=1, head_dim=8, tile=(1, 2, 2))
    cases = 0
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        ext, q, keys = (part.split() for part in line.split("|"))
        lists = M.window_lists_grouped(lay, (2, 1, 1), tuple(int(x) for x in ext))
        assert lists[int(q[0])] == [int(k) for k in keys], line
        cases += 1
    assert cases == 10


@pytest.mark.parametrize("shape,tile,r", [((5, 9, 13), (2, 4, 4), (1, 1, 2)),
                                          ((21, 30, 52), (4, 4, 4), (1, 2, 2)),
                                          ((4, 8, 8), (2, 4, 4), (0, 1, 0))])
def test_unit_groups_and_odd_extents_are_the_radius_window(shape, tile, r):
    """Groups of one tile with extents 2r+1 give the (separately pinned) radius-r window."""
    T, H, W = shape
    lay = Layout(T=T, H=H, W=W, heads=1, head_dim=8, tile=tile)
    ext = tuple(2 * x + 1 for x in r)
    assert M.window_lists_grouped(lay, (1, 1, 1), ext) == M.window_lists(lay, *r)


def _axis_pairs(n, g, e):
    """Sum over the n tiles of an axis of the key tiles its group's window covers."""
    ng = -(-n // g)
    total = 0
    for i in range(n):
        lo = max(i // g - (e - 1) // 2, 0)
        hi = min(i // g - (e - 1) // 2 + e - 1, ng - 1)
        total += min((hi + 1) * g, n) - lo * g
    return total


@pytest.mark.parametrize("ext", [(6, 6, 6), (6, 6, 1), (3, 3, 1), (2, 1, 4)])
def test_pair_count_is_the_product_over_axes(ext):
    """The window is a box in group coordinates, so the (query, key) tile pairs
    factor over the axes: 480p latent with (6,8,8) big tiles built from (1,8,8) tiles."""
    lay = Layout(T=21, H=30, W=52, heads=1, head_dim=8, tile=(1, 8, 8))
    lists = M.window_lists_grouped(lay, (6, 1, 1), ext)
    nt, nh, nw = lay.tile_grid
    expect = _axis_pairs(nt, 6, ext[0]) * _axis_pairs(nh, 1, ext[1]) * _axis_pairs(nw, 1, ext[2])
    assert sum(len(x) for x in lists) == expect
    for row in lists:
        assert row == sorted(set(row))


def _tiled(lay, rng, B=1, scale=3.0):
    x = (rng.standard_normal((B, lay.n_tokens, lay.heads, lay.head_dim)) * scale).astype(np.float32)
    return L.permute(x, lay).astype(np.float32)


def test_grouped_quantiser_unit_groups_equal_per_tile():
    lay = Layout(T=5, H=9, W=13, heads=2, head_dim=16, tile=(1, 4, 4))
    x = _tiled(lay, np.random.default_rng(3))
    c1, s1 = F.quantize_tiles(x, lay)
    c2, s2 = F.quantize_tiles_grouped(x, lay, (1, 1, 1))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_grouped_quantiser_scale_is_the_group_max():
    """Scales are monotonic in the absmax, so a group's scale is the largest
    per-tile scale of its members, and the member holding the group's absmax
    gets exactly its per-tile codes (its own absmax is the group's)."""
    lay = Layout(T=7, H=9, W=13, heads=2, head_dim=16, tile=(1, 4, 4))
    x = _tiled(lay, np.random.default_rng(4))
    c1, s1 = F.quantize_tiles(x, lay)
    group = (3, 1, 2)
    c2, s2 = F.quantize_tiles_grouped(x, lay, group)
    C = lay.tile_tokens
    groups = {}
    for t in range(lay.n_tiles):
        a, b, c = L.tile_coords(lay, t)
        groups.setdefault((a // 3, b, c // 2), []).append(t)
    assert len(groups) == 3 * 3 * 2
    for members in groups.values():
        for h in range(lay.heads):
            top = max(members, key=lambda t: s1[0, h, t])
            for t in members:
                assert s2[0, h, t] == s1[0, h, top]
            assert np.array_equal(c2[0, h, top * C:(top + 1) * C], c1[0, h, top * C:(top + 1) * C])


def test_grouped_quantiser_ignores_pads_and_bounds_error():
    """Pad rows never enter the absmax; dequantised values stay within half an
    e4m3 step (2^-4 relative for normals, 2^-10 * scale absolute below)."""
    lay = Layout(T=7, H=9, W=13, heads=1, head_dim=16, tile=(1, 4, 4))
    x = _tiled(lay, np.random.default_rng(5))
    pad = L.token_order(lay) < 0
    assert pad.any()
    x2 = x.copy()
    x2[:, :, pad] = 1e6
    c1, s1 = F.quantize_tiles_grouped(x, lay, (3, 2, 1))
    c2, s2 = F.quantize_tiles_grouped(x2, lay, (3, 2, 1))
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1[:, :, ~pad], c2[:, :, ~pad]) and not c2[:, :, pad].any()
    deq = F.dequantize_tiles(c1, s1, lay)
    sc = np.repeat(s1, lay.tile_tokens, axis=2)[..., None].astype(np.float64)
    err = np.abs(deq - x)[:, :, ~pad]
    bound = np.maximum(np.abs(x)[:, :, ~pad] * 2.0 ** -4, sc[:, :, ~pad] * 2.0 ** -10)
    assert (err <= bound * (1 + 1e-6)).all()
