"""Pins for the oracle's token layout (permute / unpermute)."""
import numpy as np
import pytest

from oracle import layout as L
from oracle.layout import Layout
from synth import CONFIGS
from tests.conftest import read_golden


def _layout_of(cfg, heads=None, d=None):
    return Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=heads or cfg.heads, head_dim=d or cfg.head_dim,
                  kind=cfg.kind, tile=cfg.tile, stride=cfg.stride)


@pytest.mark.parametrize("line", read_golden("permute_orders.txt"))
def test_golden_orders(line):
    spec, expected = line.split(":")
    f = spec.split()
    kind = f[0]
    T, H, W, tt, th, tw, sh, sw = map(int, f[1:])
    lay = Layout(T=T, H=H, W=W, heads=1, head_dim=1, kind=kind, tile=(tt, th, tw), stride=(sh, sw))
    assert L.token_order(lay).tolist() == [int(x) for x in expected.split()]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_order_is_bijection_on_real_tokens(name):
    cfg = CONFIGS[name]
    lay = _layout_of(cfg)
    order = L.token_order(lay)
    real = order[order >= 0]
    assert np.array_equal(np.sort(real), np.arange(lay.n_tokens))
    assert order.size == lay.n_padded
    assert lay.n_padded % lay.tile_tokens == 0


def test_padded_sizes_of_workloads():
    # padded token counts implied by padding each axis to the tile extent
    expect = {"tiny_window_f32": (256, 8), "topk32_16x32x32": (16384, 256),
              "window_480p": (39936, 624), "skiparse_768p": (80640, 1260),
              "fp8_topp_720p": (92160, 1440)}
    for name, (npad, ntiles) in expect.items():
        lay = _layout_of(CONFIGS[name])
        assert (lay.n_padded, lay.n_tiles) == (npad, ntiles), name


@pytest.mark.parametrize("name", ["tiny_window_f32", "window_480p", "fp8_topp_720p"])
def test_tile3d_positions_fall_in_their_tile_box(name):
    # independent derivation: tiled position p sits in tile p // C, whose box is
    # [a*tt, a*tt+tt) x [b*th, ...) x [c*tw, ...); within-tile offset is row-major
    cfg = CONFIGS[name]
    lay = _layout_of(cfg)
    order = L.token_order(lay)
    tt, th, tw = lay.tile
    nt, nh, nw = lay.tile_grid
    C = lay.tile_tokens
    rng = np.random.default_rng(0)
    for p in rng.integers(0, lay.n_padded, size=2000):
        tile, off = divmod(int(p), C)
        a, rem = divmod(tile, nh * nw)
        b, c = divmod(rem, nw)
        i, rem = divmod(off, th * tw)
        j, k = divmod(rem, tw)
        t, h, w = a * tt + i, b * th + j, c * tw + k
        if t < lay.T and h < lay.H and w < lay.W:
            assert order[p] == (t * lay.H + h) * lay.W + w
        else:
            assert order[p] == -1


def test_skiparse_groups_hold_one_residue():
    cfg = CONFIGS["skiparse_768p"]
    lay = _layout_of(cfg)
    order = L.token_order(lay)
    per_group = lay.tiles_per_group * lay.tile_tokens
    assert lay.tiles_per_group == 315 and per_group == 20160
    for g in range(4):
        toks = order[g * per_group:(g + 1) * per_group]
        toks = toks[toks >= 0]
        h = (toks // lay.W) % lay.H
        w = toks % lay.W
        assert np.all(h % 2 == g // 2) and np.all(w % 2 == g % 2)
        assert np.all(np.diff(toks) > 0)      # row-major inside the group


@pytest.mark.parametrize("name", list(CONFIGS))
def test_permute_unpermute_identity_and_zero_pads(name):
    cfg = CONFIGS[name]
    lay = _layout_of(cfg, heads=2, d=8)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, lay.n_tokens, 2, 8)).astype(np.float32)
    xt = L.permute(x, lay)
    assert xt.shape == (2, 2, lay.n_padded, 8)
    order = L.token_order(lay)
    assert np.all(xt[:, :, order < 0, :] == 0)
    assert np.array_equal(L.unpermute(xt, lay), x)
    # spot check the gather direction on a few positions
    for p in np.nonzero(order >= 0)[0][:50]:
        assert np.array_equal(xt[1, 0, p], x[1, order[p], 0])


def test_bf16_v_operand_order_golden_and_bijection():
    tok = L.v_operand_order_bf16()
    for line in read_golden("bf16_v_operand_order.txt"):
        p, t = (int(x) for x in line.split(":"))
        assert tok[p] == t
    assert sorted(tok.tolist()) == list(range(32))
    # each half-wave's 8 positions of a group are two runs of 4 consecutive tokens
    for ps in range(2):
        for h in range(2):
            run = tok[16 * ps + 8 * h: 16 * ps + 8 * h + 8]
            assert list(run[:4]) == list(range(run[0], run[0] + 4))
            assert list(run[4:]) == list(range(run[4], run[4] + 4))
            assert run[4] - run[0] == 8


def test_bf16_v_operand_layout_places_every_element():
    lay = L.Layout(T=5, H=9, W=13, heads=2, head_dim=16, tile=(4, 4, 4))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, lay.heads, lay.n_padded, lay.head_dim))
    y = L.v_operand_layout_bf16(x, lay)
    assert y.shape == x.shape
    tok = L.v_operand_order_bf16()
    yy = y.reshape(2, lay.heads, lay.n_tiles, 2, lay.head_dim, 32)
    for (b, h, j, k, c, p) in [(0, 0, 0, 0, 0, 0), (1, 1, lay.n_tiles - 1, 1, 15, 31), (0, 1, 3, 1, 7, 9),
                               (1, 0, 5, 0, 12, 22)]:
        assert yy[b, h, j, k, c, p] == x[b, h, 64 * j + 32 * k + tok[p], c]
    # the layout is a permutation of each tile's elements
    for j in range(lay.n_tiles):
        a = np.sort(x[:, :, 64 * j: 64 * (j + 1)].reshape(2, lay.heads, -1), axis=-1)
        bb = np.sort(y[:, :, 64 * j: 64 * (j + 1)].reshape(2, lay.heads, -1), axis=-1)
        assert np.array_equal(a, bb)
