"""Gradients of the block-sparse attention with respect to Q, K and V, in fp64.

TEST INFRASTRUCTURE ONLY (part of the oracle package; see its header).

The pages train through this attention: VSA is a trainable sparse attention
used to pretrain and fine-tune video DiTs (VSA page, Research Type and
Experiment Setup rows), and FPSAttention trains jointly with FP8 and tile
sparsity (FPSAttention, "Approach" and the training-loss rows of its results
table). They print no formula for the backward pass; the gradients of the
forward's definition (oracle.attention) follow from the chain rule and are
written out here directly. For real query token i with key set A(i), scores
S_ij = sigma q_i.k_j and weights P_ij = softmax_{j in A(i)} S_ij, and an
upstream gradient dO_i of the output O_i = sum_j P_ij v_j:
    dV_j  = sum_{i : j in A(i)} P_ij dO_i
    dP_ij = dO_i . v_j
    dS_ij = P_ij (dP_ij - sum_{l in A(i)} P_il dP_il)
    dQ_i  = sigma sum_{j in A(i)} dS_ij k_j
    dK_j  = sigma sum_{i : j in A(i)} dS_ij q_i
Readings: pad query rows and query rows with an empty key set contribute
nothing and get dQ = 0; pad key rows get dK = dV = 0 (they are in no A(i)).
No online softmax and no recomputation tricks: each query tile's weights are
formed in full from its key set.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Tuple

import numpy as np

from .attention import ListFn, attend_block
from .layout import Layout, token_order


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, lay: Layout,
                       lists: ListFn, sigma: float,
                       items: Optional[Iterable[Tuple[int, int, int]]] = None):
    """dQ, dK, dV (fp64) of the block-sparse attention on tiled tensors [B, heads, N_pad, d].

    ``lists(b, h, qt)`` gives the key tiles of query tile qt, as for the
    forward. ``items`` restricts the work to some (b, head, q_tile) triples:
    dQ rows of other query tiles are NaN, and dK / dV hold the contributions
    of the listed items only, so a key tile's rows are complete when every
    query tile whose list holds it is among the items.
    """
    B = q.shape[0]
    C = lay.tile_tokens
    order = token_order(lay).reshape(lay.n_tiles, C)
    real = order >= 0
    dQ = np.full(q.shape, np.nan)
    dK = np.zeros(k.shape)
    dV = np.zeros(v.shape)
    if items is None:
        items = [(b, h, t) for b in range(B) for h in range(lay.heads) for t in range(lay.n_tiles)]
    for b, h, qt in items:
        rows = slice(qt * C, (qt + 1) * C)
        key_pos: List[int] = []
        for kt in lists(b, h, qt):
            key_pos.extend(kt * C + np.nonzero(real[kt])[0])
        key_pos = np.asarray(key_pos, dtype=np.int64)
        dq = np.zeros((C, lay.head_dim))
        qi = q[b, h, rows].astype(np.float64)
        live = real[qt]
        if key_pos.size and live.any():
            kj = k[b, h, key_pos].astype(np.float64)
            vj = v[b, h, key_pos].astype(np.float64)
            _, _, p = attend_block(qi[live], kj, vj, sigma)
            do = dout[b, h, rows].astype(np.float64)[live]
            dp = do @ vj.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[live] = sigma * (ds @ kj)
            np.add.at(dK[b, h], key_pos, sigma * (ds.T @ qi[live]))
            np.add.at(dV[b, h], key_pos, p.T @ do)
        dQ[b, h, rows] = dq
    return dQ, dK, dV


def transposed_lists(lay: Layout, lists: ListFn, B: int = 1):
    """For every (b, head, key tile j): the ascending query tiles whose list holds j."""
    out = [[[[] for _ in range(lay.n_tiles)] for _ in range(lay.heads)] for _ in range(B)]
    for b in range(B):
        for h in range(lay.heads):
            for qt in range(lay.n_tiles):
                for kt in sorted(set(int(t) for t in lists(b, h, qt))):
                    out[b][h][kt].append(qt)
    return out


def key_tile_gradients(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, lay: Layout,
                       lists: ListFn, sigma: float, b: int, h: int, kt: int, query_tiles=None):
    """dK and dV rows [C, d] of key tile kt in (b, head h), from the same
    definition as attention_backward restricted to that tile's columns: for
    each query tile whose list holds kt, the weights P and the row sums
    sum_l P_il dP_il are formed over the tile's full key set, and only the
    columns of kt are accumulated. ``query_tiles`` (the query tiles whose
    lists hold kt) is computed when not given.
    """
    C = lay.tile_tokens
    order = token_order(lay).reshape(lay.n_tiles, C)
    real = order >= 0
    if query_tiles is None:
        query_tiles = [qt for qt in range(lay.n_tiles) if kt in set(int(t) for t in lists(b, h, qt))]
    dk = np.zeros((C, lay.head_dim))
    dv = np.zeros((C, lay.head_dim))
    own = np.nonzero(real[kt])[0]
    for qt in query_tiles:
        live = real[qt]
        if not live.any():
            continue
        rows = slice(qt * C, (qt + 1) * C)
        key_pos: List[int] = []
        for t in lists(b, h, qt):
            key_pos.extend(t * C + np.nonzero(real[t])[0])
        key_pos = np.asarray(key_pos, dtype=np.int64)
        qi = q[b, h, rows].astype(np.float64)[live]
        do = dout[b, h, rows].astype(np.float64)[live]
        kj = k[b, h, key_pos].astype(np.float64)
        vj = v[b, h, key_pos].astype(np.float64)
        _, _, p = attend_block(qi, kj, vj, sigma)
        rowsum = (p * (do @ vj.T)).sum(axis=1, keepdims=True)
        for pos in own:
            cols = np.nonzero(key_pos == kt * C + pos)[0]
            for c in cols:
                pc = p[:, c]
                dpc = do @ vj[c]
                dsc = pc * (dpc - rowsum[:, 0])
                dk[pos] += sigma * (dsc @ qi)
                dv[pos] += pc @ do
    return dk, dv
