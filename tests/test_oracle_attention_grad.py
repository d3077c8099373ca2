"""Pins for the oracle's attention gradients (oracle.attention_grad).

Each pin is independent of the gradient formulas: central finite differences
of the (separately pinned) forward, torch autograd through a dense masked
softmax attention, and closed forms / conservation laws of the softmax
Jacobian.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import attention_grad as G
from oracle import layout as L
from oracle import masks as M
from oracle.layout import Layout


def _random_lists(lay, B, rng, p=0.5, empty=((0, 0, 1),)):
    """Per-(b, head, q tile) ascending random key-tile subsets; some rows empty."""
    table = []
    for b in range(B):
        per_h = []
        for h in range(lay.heads):
            rows = []
            for qt in range(lay.n_tiles):
                if (b, h, qt) in empty:
                    rows.append([])
                    continue
                row = [kt for kt in range(lay.n_tiles) if rng.random() < p]
                rows.append(row or [int(rng.integers(lay.n_tiles))])
            per_h.append(rows)
        table.append(per_h)
    return table


def _tiled_inputs(lay, B, rng, zero_pads=True):
    shape = (B, lay.heads, lay.n_padded, lay.head_dim)
    q, k, v, do = (rng.standard_normal(shape) for _ in range(4))
    if zero_pads:
        pad = L.token_order(lay) < 0
        for x in (q, k, v, do):
            x[:, :, pad] = 0.0
    return q, k, v, do


def _loss(q, k, v, do, lay, lists, sigma):
    O, _ = A.attention(q, k, v, lay, lists, sigma)
    return float((O * do).sum())


def test_matches_central_finite_differences():
    """Every element of dQ, dK and dV against (L(x+h) - L(x-h)) / 2h of the forward."""
    lay = Layout(T=1, H=3, W=5, heads=2, head_dim=4, tile=(1, 2, 2))   # 6 tiles, pads
    B = 1
    rng = np.random.default_rng(7)
    lists = A.routed_lists(_random_lists(lay, B, rng))
    q, k, v, do = _tiled_inputs(lay, B, rng, zero_pads=False)   # pads must get 0 too
    sigma = 0.7
    dQ, dK, dV = G.attention_backward(q, k, v, do, lay, lists, sigma)
    h = 1e-5
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(q, k, v, do, lay, lists, sigma)
            x[idx] = keep - h
            dn = _loss(q, k, v, do, lay, lists, sigma)
            x[idx] = keep
            fd[idx] = (up - dn) / (2 * h)
        assert np.abs(fd - g).max() < 1e-7, name


def _dense_mask(lay, lists, b, h):
    C = lay.tile_tokens
    real = L.token_order(lay) >= 0
    m = np.zeros((lay.n_padded, lay.n_padded), dtype=bool)
    for qt in range(lay.n_tiles):
        for kt in lists(b, h, qt):
            m[qt * C:(qt + 1) * C, kt * C:(kt + 1) * C] = True
    return m & real[:, None] & real[None, :]


def test_matches_torch_autograd_of_dense_masked_attention():
    """Library cross-check: softmax attention with an explicit token mask, fp64 autograd."""
    lay = Layout(T=5, H=6, W=7, heads=2, head_dim=16, tile=(2, 2, 2))
    B = 2
    rng = np.random.default_rng(11)
    table = M.window_lists(lay, 1, 0, 1)
    lists = A.shared_lists(table)
    q, k, v, do = _tiled_inputs(lay, B, rng)
    sigma = 0.3
    dQ, dK, dV = G.attention_backward(q, k, v, do, lay, lists, sigma)
    for b in range(B):
        for h in range(lay.heads):
            mask = torch.from_numpy(_dense_mask(lay, lists, b, h))
            tq, tk, tv = (torch.tensor(x[b, h], requires_grad=True) for x in (q, k, v))
            s = sigma * tq @ tk.T
            s = s.masked_fill(~mask, -math.inf)
            p = torch.softmax(s, dim=1)
            p = torch.where(mask.any(dim=1, keepdim=True), p, torch.zeros_like(p))
            o = p @ tv
            (o * torch.from_numpy(do[b, h])).sum().backward()
            assert np.allclose(dQ[b, h], tq.grad.numpy(), atol=1e-12, rtol=1e-10)
            assert np.allclose(dK[b, h], tk.grad.numpy(), atol=1e-12, rtol=1e-10)
            assert np.allclose(dV[b, h], tv.grad.numpy(), atol=1e-12, rtol=1e-10)


@pytest.fixture(scope="module")
def window_case():
    lay = Layout(T=5, H=6, W=7, heads=2, head_dim=8, tile=(2, 2, 2))
    B = 1
    rng = np.random.default_rng(5)
    lists = A.routed_lists(_random_lists(lay, B, rng, p=0.4, empty=((0, 1, 3),)))
    q, k, v, do = _tiled_inputs(lay, B, rng)
    return lay, B, lists, q, k, v, do


def test_conservation_laws(window_case):
    """Rows of the softmax Jacobian sum to zero: sum_j dK_j = 0; rows of P sum to
    one: sum_j dV_j = sum of dO over real query rows with a non-empty key set."""
    lay, B, lists, q, k, v, do = window_case
    dQ, dK, dV = G.attention_backward(q, k, v, do, lay, lists, 0.45)
    real = L.token_order(lay) >= 0
    C = lay.tile_tokens
    for h in range(lay.heads):
        assert np.abs(dK[0, h].sum(axis=0)).max() < 1e-12 * max(1.0, np.abs(dK[0, h]).sum())
        live = np.zeros(lay.n_padded, dtype=bool)
        for qt in range(lay.n_tiles):
            if any(real[kt * C:(kt + 1) * C].any() for kt in lists(0, h, qt)):
                live[qt * C:(qt + 1) * C] = real[qt * C:(qt + 1) * C]
        assert np.allclose(dV[0, h].sum(axis=0), do[0, h][live].sum(axis=0), atol=1e-11)


def test_zero_scale_closed_form(window_case):
    """sigma = 0: uniform weights, so dQ = dK = 0 and dV_j = sum_{i: j in A(i)} dO_i / |A(i)|."""
    lay, B, lists, q, k, v, do = window_case
    dQ, dK, dV = G.attention_backward(q, k, v, do, lay, lists, 0.0)
    assert np.abs(dQ).max() == 0.0 and np.abs(dK).max() == 0.0
    real = L.token_order(lay) >= 0
    C = lay.tile_tokens
    ref = np.zeros_like(dV)
    for h in range(lay.heads):
        for i in range(lay.n_padded):
            if not real[i]:
                continue
            keys = [kt * C + r for kt in lists(0, h, i // C) for r in range(C) if real[kt * C + r]]
            for j in keys:
                ref[0, h, j] += do[0, h, i] / len(keys)
    assert np.allclose(dV, ref, atol=1e-13)


def test_constant_values_give_no_score_gradient(window_case):
    """V rows all equal: O does not depend on the weights, so dQ = dK = 0."""
    lay, B, lists, q, k, v, do = window_case
    vc = np.broadcast_to(np.arange(lay.head_dim, dtype=np.float64), v.shape).copy()
    dQ, dK, _ = G.attention_backward(q, k, vc, do, lay, lists, 0.8)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12


def test_pads_get_zero_gradients(window_case):
    lay, B, lists, q, k, v, do = window_case
    dQ, dK, dV = G.attention_backward(q, k, v, do, lay, lists, 0.45)
    pad = L.token_order(lay) < 0
    assert pad.any()
    for x in (dQ, dK, dV):
        assert np.abs(x[:, :, pad]).max() == 0.0


def test_items_restriction_and_transposed_lists(window_case):
    """dQ rows of chosen items and the dK / dV rows of a key tile whose attending
    query tiles are all chosen equal the full computation."""
    lay, B, lists, q, k, v, do = window_case
    full = G.attention_backward(q, k, v, do, lay, lists, 0.45)
    tl = G.transposed_lists(lay, lists, B)
    C = lay.tile_tokens
    for h in range(lay.heads):
        for kt in (0, lay.n_tiles // 2, lay.n_tiles - 1):
            qts = tl[0][h][kt]
            for qt in qts:
                assert kt in lists(0, h, qt)
            part = G.attention_backward(q, k, v, do, lay, lists, 0.45,
                                        items=[(0, h, qt) for qt in qts])
            rows = slice(kt * C, (kt + 1) * C)
            assert np.array_equal(part[1][0, h, rows], full[1][0, h, rows])
            assert np.array_equal(part[2][0, h, rows], full[2][0, h, rows])
            for qt in qts:
                r = slice(qt * C, (qt + 1) * C)
                assert np.array_equal(part[0][0, h, r], full[0][0, h, r])


def test_key_tile_gradients_match_full(window_case):
    """The one-key-tile form used for sampled checks at full size equals the
    rows of the full backward."""
    lay, B, lists, q, k, v, do = window_case
    _, dK, dV = G.attention_backward(q, k, v, do, lay, lists, 0.45)
    C = lay.tile_tokens
    for h in range(lay.heads):
        for kt in (0, 5, lay.n_tiles - 1):
            dk, dv = G.key_tile_gradients(q, k, v, do, lay, lists, 0.45, 0, h, kt)
            assert np.allclose(dk, dK[0, h, kt * C:(kt + 1) * C], atol=1e-12, rtol=1e-10)
            assert np.allclose(dv, dV[0, h, kt * C:(kt + 1) * C], atol=1e-12, rtol=1e-10)
