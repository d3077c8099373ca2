"""Adaptive block selection: tile mean-pool, coarse scores, top-k / top-p.

Follows:
  * VSA page ("Faster Video Diffusion with Trainable Sparse Attention"),
    Research Type row: trainable sparse attention that picks key blocks per
    query block (coarse stage then fine stage);
  * FVAttn summary page, "Summary": Top-p routing with a Top-k safety floor
    over video-aware blocks, per head.

The pages give neither formulas nor tie rules. Readings taken:
  * pool: mean over the tile's real (non-pad) tokens, from the bf16 values,
    in fp64 here; a tile without real tokens takes no part in routing;
  * coarse score s_ij = coarse_scale * <qbar_i, kbar_j> over real key tiles,
    coarse_scale = 1/sqrt(d) in the workloads (same scale as the fine stage);
  * top-k: descending score, lower key-tile index first on exact ties; if
    fewer than k real tiles exist, all of them are kept;
  * top-p: p_ij = softmax_j(s_ij) over real key tiles; keep the shortest
    prefix of the descending order whose mass reaches p (the tile that crosses
    p is kept); then count = min(max(count, k_floor), #real tiles);
  * the kept set is returned in ascending key-tile order.
"""
from __future__ import annotations

from typing import List

import numpy as np

from .layout import Layout, token_order


def pool_tiles(x_tiled: np.ndarray, lay: Layout) -> np.ndarray:
    """Mean over real tokens of each tile: [B, heads, N_pad, d] -> [B, heads, n_tiles, d].

    Tiles without real tokens get NaN (they are excluded from routing).
    """
    order = token_order(lay).reshape(lay.n_tiles, lay.tile_tokens)
    B = x_tiled.shape[0]
    out = np.full((B, lay.heads, lay.n_tiles, lay.head_dim), np.nan)
    xt = x_tiled.astype(np.float64).reshape(B, lay.heads, lay.n_tiles, lay.tile_tokens,
                                             lay.head_dim)
    for t in range(lay.n_tiles):
        real = order[t] >= 0
        if real.any():
            out[:, :, t, :] = xt[:, :, t, real, :].mean(axis=2)
    return out


def coarse_scores(qbar: np.ndarray, kbar: np.ndarray, coarse_scale: float) -> np.ndarray:
    """s[b, h, i, j] = coarse_scale * <qbar_i, kbar_j>.

    -inf where key tile j has no real token; a whole row is NaN where query
    tile i has no real token.
    """
    s = coarse_scale * np.matmul(qbar, np.swapaxes(kbar, -1, -2))
    bad_key = np.isnan(kbar).any(axis=-1)                 # [B, heads, n_tiles]
    bad_query = np.isnan(qbar).any(axis=-1)
    s = np.where(bad_key[:, :, None, :], -np.inf, s)
    s = np.where(bad_query[:, :, :, None], np.nan, s)
    return s


def _descending(row: np.ndarray) -> List[int]:
    """Key tiles with finite score, by descending score then ascending index."""
    idx = [j for j in range(row.size) if np.isfinite(row[j])]
    return sorted(idx, key=lambda j: (-row[j], j))


def topk_row(row: np.ndarray, k: int) -> List[int]:
    keep = _descending(row)[:k]
    return sorted(keep)


def topp_row(row: np.ndarray, p: float, k_floor: int) -> List[int]:
    order = _descending(row)
    if not order:
        return []
    vals = np.array([row[j] for j in order])
    w = np.exp(vals - vals.max())
    probs = w / w.sum()
    cum = 0.0
    count = len(order)
    for m, pr in enumerate(probs):
        cum += pr
        if cum >= p:
            count = m + 1
            break
    count = min(max(count, k_floor), len(order))
    return sorted(order[:count])


def select_lists(scores: np.ndarray, top_k: int = 0, top_p: float = 0.0,
                 k_floor: int = 0):
    """Apply top-k (top_p <= 0) or top-p with floor to every (b, head, q-tile) row.

    Returns a nested list lists[b][h][qt] of ascending key-tile indices.
    Query tiles without real tokens get an empty list.
    """
    B, Hh, n, _ = scores.shape
    out = []
    for b in range(B):
        per_head = []
        for h in range(Hh):
            rows = []
            for i in range(n):
                row = scores[b, h, i]
                if np.isnan(row).all():
                    rows.append([])
                elif top_p > 0.0:
                    rows.append(topp_row(row, top_p, k_floor))
                else:
                    rows.append(topk_row(row, top_k))
            per_head.append(rows)
        out.append(per_head)
    return out


def route(q_tiled: np.ndarray, k_tiled: np.ndarray, lay: Layout, coarse_scale: float,
          top_k: int = 0, top_p: float = 0.0, k_floor: int = 0):
    """Pool, score and select: returns (lists[b][h][qt], scores)."""
    qbar = pool_tiles(q_tiled, lay)
    kbar = pool_tiles(k_tiled, lay)
    s = coarse_scores(qbar, kbar, coarse_scale)
    # a query tile without real tokens has NaN pooled values -> NaN scores row
    return select_lists(s, top_k=top_k, top_p=top_p, k_floor=k_floor), s


def select_lists_vectorized(scores: np.ndarray, top_k: int = 0, top_p: float = 0.0,
                            k_floor: int = 0):
    """Same rule as ``select_lists`` for many rows at once (library sort + cumsum).

    Used for full-size workloads where the per-row Python version is too slow;
    ``tests/test_oracle_routing.py`` checks that both give identical lists.
    Returns (idx int32 [..., n, n] ascending and padded with -1, cnt int32 [..., n]).
    """
    s = np.asarray(scores, dtype=np.float64)
    lead = s.shape[:-1]
    n = s.shape[-1]
    rows = s.reshape(-1, n)
    R = rows.shape[0]
    idx = np.full((R, n), -1, dtype=np.int32)
    cnt = np.zeros(R, dtype=np.int32)
    col = np.broadcast_to(np.arange(n), rows.shape)
    finite = np.isfinite(rows)
    n_valid = finite.sum(axis=1)
    q_bad = np.isnan(rows).all(axis=1)
    # descending score, ascending index; non-finite scores go last
    key = np.where(finite, -rows, np.inf)
    order = np.lexsort((col, key), axis=-1)
    for r in range(R):
        if q_bad[r] or n_valid[r] == 0:
            continue
        o = order[r, :n_valid[r]]
        if top_p > 0.0:
            v = rows[r, o]
            w = np.exp(v - v[0])
            cum = np.cumsum(w / w.sum())
            hit = np.nonzero(cum >= top_p)[0]
            c = int(hit[0]) + 1 if hit.size else int(n_valid[r])
            c = min(max(c, k_floor), int(n_valid[r]))
        else:
            c = min(top_k, int(n_valid[r]))
        keep = np.sort(o[:c])
        idx[r, :c] = keep
        cnt[r] = c
    return idx.reshape(lead + (n,)), cnt.reshape(lead)
