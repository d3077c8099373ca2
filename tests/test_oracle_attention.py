"""Pins for the oracle's block-sparse attention."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import layout as L
from oracle import masks as M
from oracle.layout import Layout
from synth import CONFIGS, make_qkv


def _brute_force(q, k, v, allowed, sigma):
    """Per-query Python loops over natural-order tokens; allowed(i, j) -> bool."""
    B, n, Hh, d = q.shape
    out = np.zeros_like(q, dtype=np.float64)
    lse = np.full((B, n, Hh), -np.inf)
    for b in range(B):
        for h in range(Hh):
            for i in range(n):
                keys = [j for j in range(n) if allowed(i, j)]
                if not keys:
                    continue
                s = [sigma * sum(float(q[b, i, h, e]) * float(k[b, j, h, e]) for e in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                z = sum(w)
                for e in range(d):
                    out[b, i, h, e] = sum(w[t] * float(v[b, keys[t], h, e]) for t in range(len(keys))) / z
                lse[b, i, h] = mx + math.log(z)
    return out, lse


def _coords(lay):
    return [(t, h, w) for t in range(lay.T) for h in range(lay.H) for w in range(lay.W)]


def _run_oracle(q, k, v, lay, lists, sigma):
    O, lse = A.attention(L.permute(q, lay), L.permute(k, lay), L.permute(v, lay), lay,
                         A.shared_lists(lists), sigma)
    order = L.token_order(lay)
    lse_nat = np.zeros((q.shape[0], lay.n_tokens, lay.heads))
    lse_nat[:, order[order >= 0], :] = np.transpose(lse[:, :, order >= 0], (0, 2, 1))
    return L.unpermute(O, lay), lse_nat


def test_tiny_workload_equals_dense_brute_force():
    cfg = CONFIGS["tiny_window_f32"]
    q, k, v = make_qkv(cfg)
    lay = Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=cfg.heads, head_dim=cfg.head_dim, tile=cfg.tile)
    lists = M.window_lists(lay, *cfg.window)
    sigma = 1.0 / math.sqrt(cfg.head_dim)
    O, lse = _run_oracle(q, k, v, lay, lists, sigma)
    # brute force on the first 24 queries only keeps the Python loops short
    ref, ref_lse = _brute_force(q, k, v, lambda i, j: i < 24, sigma)
    assert np.allclose(O[:, :24], ref[:, :24], rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[:, :24], ref_lse[:, :24], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("grid,tile,r", [((3, 5, 6), (2, 4, 4), (0, 0, 1)),
                                          ((4, 4, 8), (2, 2, 4), (1, 0, 0))])
def test_window_with_pads_equals_brute_force(grid, tile, r):
    lay = Layout(T=grid[0], H=grid[1], W=grid[2], heads=2, head_dim=4, tile=tile)
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((1, lay.n_tokens, 2, 4)) for _ in range(3))
    sigma = 0.7
    lists = M.window_lists(lay, *r)
    O, lse = _run_oracle(q, k, v, lay, lists, sigma)
    c = _coords(lay)
    tt, th, tw = tile
    allowed = lambda i, j: (abs(c[i][0] // tt - c[j][0] // tt) <= r[0] and
                            abs(c[i][1] // th - c[j][1] // th) <= r[1] and
                            abs(c[i][2] // tw - c[j][2] // tw) <= r[2])
    ref, ref_lse = _brute_force(q, k, v, allowed, sigma)
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_skiparse_equals_brute_force():
    lay = Layout(T=2, H=4, W=6, heads=1, head_dim=4, kind="skiparse2d", tile=(1, 1, 4),
                 stride=(2, 2))
    rng = np.random.default_rng(22)
    q, k, v = (rng.standard_normal((1, lay.n_tokens, 1, 4)) for _ in range(3))
    O, _ = _run_oracle(q, k, v, lay, M.skiparse_lists(lay), 0.5)
    c = _coords(lay)
    ref, _ = _brute_force(q, k, v, lambda i, j: c[i][1] % 2 == c[j][1] % 2 and
                          c[i][2] % 2 == c[j][2] % 2, 0.5)
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)


def test_matches_torch_sdpa_with_mask():
    lay = Layout(T=4, H=8, W=12, heads=3, head_dim=16, tile=(2, 4, 4))
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((1, lay.n_tokens, 3, 16)) for _ in range(3))
    r = (0, 1, 1)
    lists = M.window_lists(lay, *r)
    sigma = 0.25
    O, _ = _run_oracle(q, k, v, lay, lists, sigma)
    c = np.array(_coords(lay))
    tiles = c // np.array(lay.tile)
    mask = np.all(np.abs(tiles[:, None, :] - tiles[None, :, :]) <= np.array(r), axis=-1)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=sigma)
    assert np.allclose(O, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_zero_scale_gives_mean_of_values_over_key_set():
    lay = Layout(T=3, H=5, W=6, heads=2, head_dim=4, tile=(2, 4, 4))
    rng = np.random.default_rng(24)
    q, k, v = (rng.standard_normal((1, lay.n_tokens, 2, 4)) for _ in range(3))
    lists = M.window_lists(lay, 0, 0, 1)
    qt, kt, vt = (L.permute(x, lay) for x in (q, k, v))
    O, _ = A.attention(qt, kt, vt, lay, A.shared_lists(lists), 0.0)
    order = L.token_order(lay)
    C = lay.tile_tokens
    for t in range(lay.n_tiles):
        keys = [n for kk in lists[t] for n in order[kk * C:(kk + 1) * C] if n >= 0]
        mean = v[0, keys].mean(axis=0)                            # [heads, d]
        for p in range(t * C, (t + 1) * C):
            if order[p] >= 0:
                assert np.allclose(O[0, :, p], mean, rtol=1e-13, atol=1e-13)
            else:
                assert np.all(O[0, :, p] == 0)


def test_constant_values_give_constant_output():
    lay = Layout(T=2, H=4, W=8, heads=1, head_dim=4, tile=(1, 4, 4))
    rng = np.random.default_rng(25)
    q, k = (rng.standard_normal((1, lay.n_tokens, 1, 4)) * 3 for _ in range(2))
    v = np.full((1, lay.n_tokens, 1, 4), 2.5)
    O, _ = _run_oracle(q, k, v, lay, M.window_lists(lay, 0, 0, 1), 1.0)
    assert np.allclose(O, 2.5, rtol=1e-14, atol=1e-14)


def test_key_order_invariance_and_row_sums():
    rng = np.random.default_rng(26)
    qb = rng.standard_normal((8, 4))
    ks = rng.standard_normal((20, 4))
    vs = rng.standard_normal((20, 4))
    o1, l1, p = A.attend_block(qb, ks, vs, 0.9)
    perm = rng.permutation(20)
    o2, l2, _ = A.attend_block(qb, ks[perm], vs[perm], 0.9)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-13) and np.allclose(l1, l2, rtol=1e-13)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14) and np.all(p >= 0)


def test_empty_list_and_pad_rows():
    lay = Layout(T=3, H=4, W=4, heads=1, head_dim=4, tile=(2, 4, 4))
    rng = np.random.default_rng(27)
    x = L.permute(rng.standard_normal((1, lay.n_tokens, 1, 4)), lay)
    O, lse = A.attention(x, x, x, lay, lambda b, h, t: [] if t == 0 else [0, 1], 1.0)
    assert np.all(O[0, 0, :32] == 0) and np.all(np.isneginf(lse[0, 0, :32]))
    order = L.token_order(lay)
    pad = np.nonzero(order < 0)[0]
    assert pad.size == 16 and np.all(O[0, 0, pad] == 0) and np.all(np.isneginf(lse[0, 0, pad]))
