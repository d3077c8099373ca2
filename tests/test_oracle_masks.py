"""Pins for the oracle's fixed masks (window, Skiparse-2D, dense)."""
import numpy as np
import pytest

from oracle import layout as L
from oracle import masks as M
from oracle.layout import Layout
from synth import CONFIGS
from tests.conftest import read_golden


def _closed_form_axis(Lt, r):
    # number of (i, j) pairs with |i - j| <= r on an axis of Lt tiles:
    # Lt + 2 * sum_{k=1..min(r, Lt-1)} (Lt - k)
    return Lt + 2 * sum(Lt - k for k in range(1, min(r, Lt - 1) + 1))


@pytest.mark.parametrize("line", read_golden("window_masks.txt"))
def test_golden_window_lists(line):
    spec, expected = line.split(":")
    T, H, W, tt, th, tw, rt, rh, rw = map(int, spec.split())
    lay = Layout(T=T, H=H, W=W, heads=1, head_dim=1, tile=(tt, th, tw))
    want = [[int(x) for x in part.split()] for part in expected.split("|")]
    assert M.window_lists(lay, rt, rh, rw) == want


def test_window_counts_closed_form_480p():
    cfg = CONFIGS["window_480p"]
    lay = Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=1, head_dim=1, tile=cfg.tile)
    lists = M.window_lists(lay, *cfg.window)
    nt, nh, nw = lay.tile_grid
    assert (nt, nh, nw) == (6, 8, 13)
    total = sum(len(x) for x in lists)
    assert total == _closed_form_axis(6, 1) * _closed_form_axis(8, 2) * _closed_form_axis(13, 2)
    assert total == 16 * 34 * 59 == 32096
    assert max(len(x) for x in lists) == 75
    for row in lists:
        assert row == sorted(set(row))


def test_tiny_window_is_dense():
    cfg = CONFIGS["tiny_window_f32"]
    lay = Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=1, head_dim=1, tile=cfg.tile)
    lists = M.window_lists(lay, *cfg.window)
    assert sum(len(x) for x in lists) == 64
    assert lists == M.dense_lists(lay)


def test_skiparse_lists_768p():
    cfg = CONFIGS["skiparse_768p"]
    lay = Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=1, head_dim=1, kind="skiparse2d",
                 tile=cfg.tile, stride=cfg.stride)
    lists = M.window_lists(lay, 0, 0, 0)
    assert all(len(x) == 315 for x in lists)
    assert sum(len(x) for x in lists) * 4 == lay.n_tiles ** 2   # density exactly 1/4
    for qt in (0, 314, 315, 700, 1259):
        g = qt // 315
        assert lists[qt] == list(range(g * 315, (g + 1) * 315))
    assert M.window_lists(lay, -1, 0, 0) == M.dense_lists(lay)


def _token_mask_natural(lay, rt, rh, rw):
    """Brute force in natural coordinates: query (t,h,w) sees key (t',h',w') iff
    their tiles are within the window on every axis."""
    tt, th, tw = lay.tile
    n = lay.n_tokens
    m = np.zeros((n, n), dtype=bool)
    coords = [(t, h, w) for t in range(lay.T) for h in range(lay.H) for w in range(lay.W)]
    for i, (t, h, w) in enumerate(coords):
        for j, (t2, h2, w2) in enumerate(coords):
            m[i, j] = (abs(t // tt - t2 // tt) <= rt and abs(h // th - h2 // th) <= rh
                       and abs(w // tw - w2 // tw) <= rw)
    return m


def _token_mask_from_lists(lay, lists):
    order = L.token_order(lay)
    C = lay.tile_tokens
    n = lay.n_tokens
    m = np.zeros((n, n), dtype=bool)
    for qt, row in enumerate(lists):
        qs = order[qt * C:(qt + 1) * C]
        for kt in row:
            ks = order[kt * C:(kt + 1) * C]
            for a in qs[qs >= 0]:
                m[a, ks[ks >= 0]] = True
    return m


@pytest.mark.parametrize("grid,tile,r", [((3, 5, 6), (2, 4, 4), (0, 0, 1)),
                                          ((5, 6, 9), (2, 2, 4), (1, 1, 0)),
                                          ((4, 8, 8), (2, 4, 4), (1, 1, 1))])
def test_window_matches_token_level_brute_force(grid, tile, r):
    lay = Layout(T=grid[0], H=grid[1], W=grid[2], heads=1, head_dim=1, tile=tile)
    lists = M.window_lists(lay, *r)
    assert np.array_equal(_token_mask_from_lists(lay, lists), _token_mask_natural(lay, *r))


def test_skiparse_matches_token_level_brute_force():
    lay = Layout(T=3, H=4, W=6, heads=1, head_dim=1, kind="skiparse2d", tile=(1, 2, 2),
                 stride=(2, 2))
    lists = M.skiparse_lists(lay)
    coords = [(t, h, w) for t in range(3) for h in range(4) for w in range(6)]
    want = np.array([[(h % 2 == h2 % 2) and (w % 2 == w2 % 2) for (_, h2, w2) in coords]
                     for (_, h, w) in coords])
    assert np.array_equal(_token_mask_from_lists(lay, lists), want)
