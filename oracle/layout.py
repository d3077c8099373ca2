"""Token-grid layout: 3D tiles, Skiparse residue groups, permute / unpermute.

Follows:
  * FPSAttention summary page, "Approach": quantisation and sparsity share
    one 3D tile granularity over the latent video grid;
  * FVAttn summary page, "Summary": video-aware block organisation;
  * OSP-Next model card, "Model Summary": Skiparse-2D is a fixed-rule sparse
    pattern applied along H and W.

Readings where the pages are silent:
  * natural order is row-major (t, h, w), w fastest;
  * tiles are numbered row-major over tile coordinates, tokens row-major
    inside a tile;
  * each axis is padded at its high end to a multiple of the tile extent, and
    pad tokens hold zeros;
  * Skiparse-2D with strides (sh, sw): token (t, h, w) is in residue group
    g = (h mod sh) * sw + (w mod sw); groups are stored one after another,
    each row-major over (t, h // sh, w // sw); a group is cut into chunks of
    tile_t * tile_h * tile_w tokens and its tail chunk is padded.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass(frozen=True)
class Layout:
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    kind: str = "tile3d"           # "tile3d" | "skiparse2d"
    tile: Tuple[int, int, int] = (4, 4, 4)
    stride: Tuple[int, int] = (2, 2)
    batch: int = 1

    # ----- derived sizes -------------------------------------------------
    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def tile_tokens(self) -> int:
        return self.tile[0] * self.tile[1] * self.tile[2]

    @property
    def tile_grid(self) -> Tuple[int, int, int]:
        """Tiles per axis (3D tiles only)."""
        assert self.kind == "tile3d"
        return (_ceil_div(self.T, self.tile[0]), _ceil_div(self.H, self.tile[1]),
                _ceil_div(self.W, self.tile[2]))

    @property
    def n_groups(self) -> int:
        return self.stride[0] * self.stride[1] if self.kind == "skiparse2d" else 1

    @property
    def group_len(self) -> int:
        assert self.kind == "skiparse2d"
        sh, sw = self.stride
        return self.T * (self.H // sh) * (self.W // sw)

    @property
    def tiles_per_group(self) -> int:
        if self.kind == "tile3d":
            return self.n_tiles
        return _ceil_div(self.group_len, self.tile_tokens)

    @property
    def n_tiles(self) -> int:
        if self.kind == "tile3d":
            a, b, c = self.tile_grid
            return a * b * c
        return self.n_groups * self.tiles_per_group

    @property
    def n_padded(self) -> int:
        return self.n_tiles * self.tile_tokens

    def validate(self) -> None:
        if self.kind == "skiparse2d":
            sh, sw = self.stride
            if self.H % sh or self.W % sw:
                raise ValueError("Skiparse-2D needs H and W divisible by the strides")
        elif self.kind != "tile3d":
            raise ValueError(self.kind)


def token_order(lay: Layout) -> np.ndarray:
    """Natural token index held at each position of the tiled order (-1 = pad).

    Built with explicit loops over tiles and the tokens inside each tile, so
    the order can be read off against the rules in the module docstring.
    """
    lay.validate()
    order: List[int] = []
    T, H, W = lay.T, lay.H, lay.W
    if lay.kind == "tile3d":
        tt, th, tw = lay.tile
        nt, nh, nw = lay.tile_grid
        for a in range(nt):
            for b in range(nh):
                for c in range(nw):
                    for i in range(tt):
                        for j in range(th):
                            for k in range(tw):
                                t, h, w = a * tt + i, b * th + j, c * tw + k
                                if t < T and h < H and w < W:
                                    order.append((t * H + h) * W + w)
                                else:
                                    order.append(-1)
    else:
        sh, sw = lay.stride
        per_group = lay.tiles_per_group * lay.tile_tokens
        for g in range(lay.n_groups):
            rh, rw = g // sw, g % sw
            members = []
            for t in range(T):
                for hh in range(H // sh):
                    for ww in range(W // sw):
                        h, w = hh * sh + rh, ww * sw + rw
                        members.append((t * H + h) * W + w)
            members += [-1] * (per_group - len(members))
            order.extend(members)
    out = np.asarray(order, dtype=np.int64)
    assert out.size == lay.n_padded
    return out


def tile_valid_counts(lay: Layout) -> np.ndarray:
    """Number of real (non-pad) tokens in every tile."""
    order = token_order(lay).reshape(lay.n_tiles, lay.tile_tokens)
    return (order >= 0).sum(axis=1)


def tile_coords(lay: Layout, tile: int) -> Tuple[int, int, int]:
    """(tile_t, tile_h, tile_w) coordinates of a 3D tile index."""
    nt, nh, nw = lay.tile_grid
    return tile // (nh * nw), (tile // nw) % nh, tile % nw


def tile_group(lay: Layout, tile: int) -> int:
    """Residue group of a Skiparse tile (0 for 3D tiles)."""
    if lay.kind != "skiparse2d":
        return 0
    return tile // lay.tiles_per_group


def permute(x_nat: np.ndarray, lay: Layout) -> np.ndarray:
    """Natural [B, T*H*W, heads, d] -> tiled [B, heads, N_pad, d]; pads are 0."""
    order = token_order(lay)
    B = x_nat.shape[0]
    out = np.zeros((B, lay.heads, lay.n_padded, lay.head_dim), dtype=x_nat.dtype)
    real = order >= 0
    # out[b, h, p, :] = x_nat[b, order[p], h, :] for every real position p
    out[:, :, real, :] = np.transpose(x_nat[:, order[real], :, :], (0, 2, 1, 3))
    return out


def unpermute(x_tiled: np.ndarray, lay: Layout) -> np.ndarray:
    """Tiled [B, heads, N_pad, d] -> natural [B, T*H*W, heads, d]; pads dropped."""
    order = token_order(lay)
    B = x_tiled.shape[0]
    out = np.zeros((B, lay.n_tokens, lay.heads, lay.head_dim), dtype=x_tiled.dtype)
    real = order >= 0
    out[:, order[real], :, :] = np.transpose(x_tiled[:, :, real, :], (0, 2, 1, 3))
    return out


def v_operand_order_bf16() -> np.ndarray:
    """Token of a 32-token block held at each position p (0..31) of the bf16
    P.V operand.

    Layout reading (the pages are silent on layouts; the P.V product of the
    flash-style forward takes V transposed): in each 16-position group ps,
    position 16 ps + 8 h + i holds token 16 ps + 8 (i div 4) + 4 h + (i mod 4),
    with h in 0..1 and i in 0..7.
    """
    tok = np.empty(32, dtype=np.int64)
    for ps in range(2):
        for h in range(2):
            for i in range(8):
                tok[16 * ps + 8 * h + i] = 16 * ps + 8 * (i // 4) + 4 * h + (i % 4)
    return tok


def v_operand_layout_bf16(x_tiled: np.ndarray, lay: Layout) -> np.ndarray:
    """A tiled tensor [B, heads, N_pad, d] of 64-token tiles stored, per tile,
    as two 32-token blocks each channel-major in the bf16 P.V operand order:
    element (block k, channel c, position p) of tile j sits at
    ((2 j + k) * d + c) * 32 + p of its (b, head) slice and holds channel c of
    token 32 k + v_operand_order_bf16()[p] of the tile.
    """
    assert lay.tile_tokens == 64
    B, d = x_tiled.shape[0], lay.head_dim
    x = np.asarray(x_tiled).reshape(B, lay.heads, lay.n_tiles, 2, 32, d)
    x = np.swapaxes(x[:, :, :, :, v_operand_order_bf16(), :], -1, -2)   # [.., block, channel, position]
    return np.ascontiguousarray(x).reshape(B, lay.heads, lay.n_padded, d)
