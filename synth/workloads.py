"""The five synthetic workloads and their seeded Q/K/V generator.

Grids follow the Wan2.1-class latent shapes the pages measure on: 81 frames
give T = 21 latent frames, and 480p / 720p / 768p give H x W = 30 x 52,
45 x 80 and 48 x 80 latent positions; the (16, 32, 32) latent of the VSA page
("Faster Video Diffusion with Trainable Sparse Attention", Open Datasets row)
is the adaptive top-k case. Random Q/K/V stand in for the activations a
trained DiT would produce on VBench-style prompts; no dataset item is used.

Recipe (identical for every consumer):
  rng = numpy.random.default_rng(seed)
  (top-p workload only) sigma_h ~ U[0.3, 1.5] per head, drawn first;
  for Q, K, V in turn:
     base   = rng.standard_normal((B, T, H, W, heads, d), float32)
     offset = rng.standard_normal((B, heads, nT, nH, nW, d), float32) * sigma
  every token gets the offset of the natural-grid 3D tile it falls in
  (tile extents = the workload's tile; partial tiles at the high end);
  bf16 workloads are then rounded to bf16 with round-to-nearest-even.
The returned arrays are in natural token order, [B, T*H*W, heads, d].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16" (input / permute dtype)
    kind: str                  # "tile3d" or "skiparse2d"
    tile: Tuple[int, int, int]  # 3D tile extents (t, h, w); skiparse: product = chunk tokens
    mask: str                  # "window" | "topk" | "topp" | "skiparse"
    seed: int
    window: Tuple[int, int, int] = (0, 0, 0)
    top_k: int = 0
    top_p: float = 0.0
    k_floor: int = 0
    stride: Tuple[int, int] = (1, 1)
    dense_every: int = 0        # hybrid: one dense layer in this many
    fp8: bool = False
    offset_std: float = 0.5
    head_std_range: Optional[Tuple[float, float]] = None
    batch: int = 1
    description: str = ""

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W


CONFIGS = {
    "tiny_window_f32": Workload(
        name="tiny_window_f32", T=4, H=8, W=8, heads=2, head_dim=64, dtype="f32",
        kind="tile3d", tile=(2, 4, 4), mask="window", window=(1, 1, 1), seed=1001,
        description="4x8x8 grid, 2 heads, d=64, fp32, 2x4x4 tiles, +-1 tile window"),
    "topk32_16x32x32": Workload(
        name="topk32_16x32x32", T=16, H=32, W=32, heads=12, head_dim=128, dtype="bf16",
        kind="tile3d", tile=(4, 4, 4), mask="topk", top_k=32, seed=1002,
        description="16x32x32 grid, 12 heads, d=128, bf16, top-32 of 256 tiles"),
    "window_480p": Workload(
        name="window_480p", T=21, H=30, W=52, heads=12, head_dim=128, dtype="bf16",
        kind="tile3d", tile=(4, 4, 4), mask="window", window=(1, 2, 2), seed=1003,
        description="21x30x52 grid padded to 24x32x52, 12 heads, window +-(1,2,2)"),
    "skiparse_768p": Workload(
        name="skiparse_768p", T=21, H=48, W=80, heads=40, head_dim=128, dtype="bf16",
        kind="skiparse2d", tile=(4, 4, 4), mask="skiparse", stride=(2, 2), dense_every=4,
        seed=1004,
        description="21x48x80 grid, 40 heads, Skiparse-2D stride (2,2), 1 dense layer in 4"),
    "fp8_topp_720p": Workload(
        name="fp8_topp_720p", T=21, H=45, W=80, heads=40, head_dim=128, dtype="bf16",
        kind="tile3d", tile=(4, 4, 4), mask="topp", top_p=0.9, k_floor=16, fp8=True,
        seed=1005, head_std_range=(0.3, 1.5),
        description="21x45x80 grid padded to 24x48x80, 40 heads, fp8 e4m3, top-p 0.9 floor 16"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _offset_field(rng, cfg: Workload, sigma_heads: np.ndarray) -> np.ndarray:
    """Per-(batch, head, natural-grid tile) offset vectors, broadcast to tokens."""
    tt, th, tw = cfg.tile
    nT = -(-cfg.T // tt)
    nH = -(-cfg.H // th)
    nW = -(-cfg.W // tw)
    off = rng.standard_normal((cfg.batch, cfg.heads, nT, nH, nW, cfg.head_dim), dtype=np.float32)
    off *= sigma_heads.astype(np.float32)[None, :, None, None, None, None]
    # token (t, h, w) takes the offset of tile (t // tt, h // th, w // tw)
    ti = np.arange(cfg.T) // tt
    hi = np.arange(cfg.H) // th
    wi = np.arange(cfg.W) // tw
    # -> [B, T, H, W, heads, d]
    o = off[:, :, ti][:, :, :, hi][:, :, :, :, wi]          # [B, heads, T, H, W, d]
    return np.moveaxis(o, 1, 4)


def make_qkv(cfg: Workload, seed: Optional[int] = None, batch: Optional[int] = None):
    """Return (q, k, v) float32 arrays [B, T*H*W, heads, d] in natural order.

    Values are bf16-representable for bf16 workloads. The same seed always
    gives the same arrays.
    """
    if batch is not None and batch != cfg.batch:
        cfg = Workload(**{**cfg.__dict__, "batch": batch})
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if cfg.head_std_range is not None:
        lo, hi = cfg.head_std_range
        sigma_heads = rng.uniform(lo, hi, size=cfg.heads)
    else:
        sigma_heads = np.full(cfg.heads, cfg.offset_std)
    out = []
    for _ in range(3):
        base = rng.standard_normal((cfg.batch, cfg.T, cfg.H, cfg.W, cfg.heads, cfg.head_dim),
                                   dtype=np.float32)
        base += _offset_field(rng, cfg, sigma_heads)
        x = base.reshape(cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim)
        if cfg.dtype == "bf16":
            x = round_to_bf16(x)
        out.append(x)
    return tuple(out)


def head_sigmas(cfg: Workload, seed: Optional[int] = None) -> np.ndarray:
    """The per-head offset std the generator uses (first draws of the stream)."""
    if cfg.head_std_range is None:
        return np.full(cfg.heads, cfg.offset_std)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lo, hi = cfg.head_std_range
    return rng.uniform(lo, hi, size=cfg.heads)


def make_grad(cfg: Workload, seed: Optional[int] = None, batch: Optional[int] = None,
              std: float = 1.0):
    """Upstream gradient dO: float32 [B, T*H*W, heads, d] in natural order,
    i.i.d. N(0, std^2) from its own stream (seed + 7919 by default), rounded
    to bf16 for bf16 workloads."""
    b = cfg.batch if batch is None else batch
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 7919)
    x = rng.standard_normal((b, cfg.n_tokens, cfg.heads, cfg.head_dim), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_to_bf16(x) if cfg.dtype == "bf16" else x
