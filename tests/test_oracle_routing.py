"""Pins for the oracle's adaptive routing (pool, coarse score, top-k, top-p)."""
import math

import numpy as np
import pytest

from oracle import layout as L
from oracle import routing as R
from oracle.layout import Layout
from tests.conftest import read_golden


@pytest.mark.parametrize("line", read_golden("routing_rows.txt"))
def test_golden_rows(line):
    spec, scores, expected = line.split(":")
    mode, param, floor = spec.split()
    row = np.array([float(x) for x in scores.split()])
    want = [int(x) for x in expected.split()]
    if mode == "topk":
        assert R.topk_row(row, int(param)) == want
    else:
        assert R.topp_row(row, float(param), int(floor)) == want


def test_pool_brute_force_with_pads():
    lay = Layout(T=3, H=5, W=6, heads=2, head_dim=3, tile=(2, 4, 4))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, lay.n_tokens, 2, 3))
    pooled = R.pool_tiles(L.permute(x, lay), lay)
    tt, th, tw = lay.tile
    nt, nh, nw = lay.tile_grid
    for tile in range(lay.n_tiles):
        a, b, c = tile // (nh * nw), (tile // nw) % nh, tile % nw
        for h in range(2):
            acc = [0.0, 0.0, 0.0]
            cnt = 0
            for t in range(a * tt, min(a * tt + tt, lay.T)):
                for y in range(b * th, min(b * th + th, lay.H)):
                    for w in range(c * tw, min(c * tw + tw, lay.W)):
                        n = (t * lay.H + y) * lay.W + w
                        for e in range(3):
                            acc[e] += x[0, n, h, e]
                        cnt += 1
            assert np.allclose(pooled[0, h, tile], [v / cnt for v in acc], rtol=1e-13, atol=1e-13)


def test_scores_are_scaled_dot_products():
    rng = np.random.default_rng(4)
    qb = rng.standard_normal((1, 1, 3, 4))
    kb = rng.standard_normal((1, 1, 5, 4))
    kb[0, 0, 2] = np.nan                       # key tile with no real token
    s = R.coarse_scores(qb, kb, 0.5)
    for i in range(3):
        for j in range(5):
            if j == 2:
                assert s[0, 0, i, j] == -np.inf
            else:
                want = 0.5 * sum(qb[0, 0, i, e] * kb[0, 0, j, e] for e in range(4))
                assert math.isclose(s[0, 0, i, j], want, rel_tol=1e-13, abs_tol=1e-13)


def test_topk_equals_stable_argsort():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        row = np.round(rng.standard_normal(n), 1)          # rounding forces ties
        k = int(rng.integers(1, 45))
        order = np.lexsort((np.arange(n), -row))          # primary -score, then index
        assert R.topk_row(row, k) == sorted(order[:k].tolist())


def test_topp_prefix_properties():
    rng = np.random.default_rng(6)
    for _ in range(300):
        n = int(rng.integers(1, 60))
        row = rng.standard_normal(n) * rng.uniform(0.1, 5.0)
        p = float(rng.uniform(0.05, 0.99))
        floor = int(rng.integers(0, 20))
        kept = R.topp_row(row, p, floor)
        probs = np.exp(row - row.max())
        probs /= probs.sum()
        order = np.lexsort((np.arange(n), -row))
        m = len(kept)
        assert kept == sorted(order[:m].tolist())             # a prefix of the order
        assert m >= min(floor, n)
        mass = probs[order[:m]].sum()
        assert mass >= p - 1e-12 or m == n
        if m > floor and m > 1:
            assert probs[order[:m - 1]].sum() < p + 1e-12     # shortest such prefix


def test_pad_query_tile_gets_empty_list():
    qb = np.full((1, 1, 2, 3), np.nan)
    qb[0, 0, 0] = 1.0
    kb = np.ones((1, 1, 2, 3))
    s = R.coarse_scores(qb, kb, 1.0)
    lists = R.select_lists(s, top_k=1)
    assert lists[0][0][1] == [] and lists[0][0][0] == [0]


def test_vectorized_selection_matches_per_row():
    rng = np.random.default_rng(8)
    s = np.round(rng.standard_normal((2, 3, 40, 40)) * 2, 1)      # ties on purpose
    s[0, 1, :, 7] = -np.inf                                          # a key tile without tokens
    s[1, 2, 5, :] = np.nan                                           # a query tile without tokens
    s[1, 2, 5, 3] = -np.inf
    for kw in ({"top_k": 5}, {"top_k": 60}, {"top_p": 0.9, "k_floor": 16},
               {"top_p": 0.5, "k_floor": 0}, {"top_p": 0.999, "k_floor": 3}):
        slow = R.select_lists(s, **kw)
        idx, cnt = R.select_lists_vectorized(s, **kw)
        for b in range(2):
            for h in range(3):
                for i in range(40):
                    c = int(cnt[b, h, i])
                    assert idx[b, h, i, :c].tolist() == slow[b][h][i]
                    assert np.all(idx[b, h, i, c:] == -1)
