"""Masked softmax attention over selected key tiles, in fp64.

Follows the pages' shared statement of the operation: a flash-style
(FlashAttention-compatible) softmax attention that only visits the key/value
tiles a block mask selects (OSP-Next wiki TL;DR and model card "Model
Summary"; FPSAttention summary "Approach"; VSA page, Research Type row;
FVAttn summary "Summary").

The result has a plain definition, so it is written out directly. For real
query token i of query tile Q(i):
    A(i)  = real key tokens inside the key tiles listed for Q(i)
    O_i   = sum_{j in A(i)} exp(sigma q_i.k_j) v_j / sum_{j in A(i)} exp(sigma q_i.k_j)
    lse_i = log sum_{j in A(i)} exp(sigma q_i.k_j)
The row maximum is subtracted before exp (exact in fp64); no online softmax.
Readings: pad query rows give O = 0 and lse = -inf; an empty A(i) gives the
same.
"""
from __future__ import annotations

from typing import Callable, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .layout import Layout, token_order

ListFn = Callable[[int, int, int], Sequence[int]]   # (b, head, q_tile) -> key tiles


def attend_block(q_blk: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, sigma: float):
    """Softmax attention of a query block against an explicit key set (fp64).

    q_blk [m, d], k_sel / v_sel [n, d]. Returns (O [m, d], lse [m], P [m, n]).
    """
    q = q_blk.astype(np.float64)
    k = k_sel.astype(np.float64)
    v = v_sel.astype(np.float64)
    if k.shape[0] == 0:
        m = q.shape[0]
        return np.zeros((m, v.shape[1])), np.full(m, -np.inf), np.zeros((m, 0))
    s = sigma * (q @ k.T)
    smax = s.max(axis=1, keepdims=True)
    e = np.exp(s - smax)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    return p @ v, (smax + np.log(z))[:, 0], p


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, lay: Layout, lists: ListFn,
              sigma: float, items: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Block-sparse attention on tiled tensors [B, heads, N_pad, d].

    ``lists(b, h, qt)`` gives the ascending key tiles of query tile qt.
    ``items`` restricts the work to some (b, head, q_tile) triples; rows not
    computed are NaN in the outputs. Returns (O, lse) in fp64.
    """
    B = q.shape[0]
    C = lay.tile_tokens
    order = token_order(lay).reshape(lay.n_tiles, C)
    real = order >= 0
    O = np.full((B, lay.heads, lay.n_padded, lay.head_dim), np.nan)
    L = np.full((B, lay.heads, lay.n_padded), np.nan)
    if items is None:
        items = [(b, h, t) for b in range(B) for h in range(lay.heads)
                 for t in range(lay.n_tiles)]
    for b, h, qt in items:
        rows = slice(qt * C, (qt + 1) * C)
        key_pos: List[int] = []
        for kt in lists(b, h, qt):
            key_pos.extend(kt * C + np.nonzero(real[kt])[0])
        key_pos = np.asarray(key_pos, dtype=np.int64)
        o, lse, _ = attend_block(q[b, h, rows], k[b, h, key_pos], v[b, h, key_pos], sigma)
        pad_q = ~real[qt]
        o[pad_q] = 0.0
        lse[pad_q] = -np.inf
        O[b, h, rows] = o
        L[b, h, rows] = lse
    return O, L


def shared_lists(table: Sequence[Sequence[int]]) -> ListFn:
    """Head- and batch-invariant lists: table[qt]."""
    return lambda b, h, qt: table[qt]


def routed_lists(table) -> ListFn:
    """Per-(batch, head) lists: table[b][h][qt]."""
    return lambda b, h, qt: table[b][h][qt]
