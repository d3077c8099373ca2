"""Block-sparse video attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libvsa.so (include/vsa.h). Every step
of the computation runs in the library's HIP kernels; this module only turns
torch tensors into device pointers, allocates outputs with torch and passes
torch's current HIP stream. There is no CPU fallback: if the library is not
built, importing the binding raises.

Pages the operations follow: "FPSAttention: Training-Aware FP8 and Sparsity
Co-Design for Fast Video Diffusion" (Approach), the "OSP-Next" model card
(Model Summary), "Faster Video Diffusion with Trainable Sparse Attention"
(Research Type row) and the FVAttn summary.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from ._lib import (EXPORTED, VSA_BF16, VSA_BF16_VOP, VSA_F32, VSA_FP8_E4M3, VSA_FP8_E4M3_VOP,
                   VSA_SKIPARSE2D, VSA_TILE3D, VsaError, VsaLayout, VsaLayoutInfo, check, lib)

__all__ = [
    "Layout", "layout_info", "tile_permute", "tile_permute_v", "tile_permute_pool", "build_mask_window",
    "build_mask_topk", "build_mask_topk_pooled",
    "quant_fp8_tiles", "quant_fp8_tiles_nat", "block_sparse_attn_fwd", "block_sparse_attn_fwd_nat",
    "block_sparse_attn_fwd_fp8_nat", "build_mask_window_grouped",
    "quant_fp8_tiles_grouped", "build_transposed_lists", "bwd_workspace_bytes",
    "block_sparse_attn_bwd", "block_sparse_attn_bwd_noalloc", "VsaError", "EXPORTED",
    "VSA_F32", "VSA_BF16", "VSA_FP8_E4M3", "VSA_FP8_E4M3_VOP", "VSA_BF16_VOP", "VSA_TILE3D",
    "VSA_SKIPARSE2D",
]


@dataclass(frozen=True)
class Layout:
    """Mirror of vsa_layout. kind: "tile3d" or "skiparse2d"."""
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    kind: str = "tile3d"
    tile: Tuple[int, int, int] = (4, 4, 4)
    stride: Tuple[int, int] = (2, 2)
    batch: int = 1

    def c(self) -> VsaLayout:
        return VsaLayout(self.batch, self.heads, self.head_dim, self.T, self.H, self.W,
                         VSA_SKIPARSE2D if self.kind == "skiparse2d" else VSA_TILE3D,
                         self.tile[0], self.tile[1], self.tile[2], self.stride[0], self.stride[1])


def layout_info(lay: Layout) -> VsaLayoutInfo:
    info = VsaLayoutInfo()
    c = lay.c()
    check(lib().vsa_layout_query(ctypes.byref(c), ctypes.byref(info)))
    return info


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_DT = {torch.float32: VSA_F32, torch.bfloat16: VSA_BF16}


# Argument checks against the layout. The C ABI takes plain pointers and has no
# way to see a tensor's dtype or size, so a wrong one here would be read or
# written as if it were right; every check below runs before the call.
def _want(t: Optional[torch.Tensor], name: str, dtypes, shape=None) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")


def _tiled_shape(lay: "Layout", info) -> tuple:
    return (lay.batch, lay.heads, int(info.n_padded), lay.head_dim)


def _natural_shape(lay: "Layout", info) -> tuple:
    return (lay.batch, int(info.n_tokens), lay.heads, lay.head_dim)


def _check_lists(lay: "Layout", info, kv_idx, kv_cnt, per_head_only=False) -> None:
    """Forward lists: int32, [n_tiles, max_kv] + [n_tiles] (one shared table) or
    [B, heads, n_tiles, max_kv] + [B, heads, n_tiles] (per (b, head)); both or neither."""
    if (kv_idx is None) != (kv_cnt is None):
        raise ValueError("kv_idx and kv_cnt must be given together")
    if kv_idx is None:
        return
    n = int(info.n_tiles)
    if kv_idx.dim() == 2 and not per_head_only:
        lead = (n,)
    elif kv_idx.dim() == 4:
        lead = (lay.batch, lay.heads, n)
    else:
        raise ValueError("kv_idx must be [n_tiles, max_kv] or [B, heads, n_tiles, max_kv]")
    if kv_idx.shape[-1] < 1:
        raise ValueError("kv_idx needs max_kv >= 1 columns")
    _want(kv_idx, "kv_idx", torch.int32, lead + (kv_idx.shape[-1],))
    _want(kv_cnt, "kv_cnt", torch.int32, lead)


def _ws_bytes(ws: torch.Tensor) -> int:
    return ws.numel() * ws.element_size()


def tile_permute(lay: Layout, src: torch.Tensor, inverse: bool = False,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Natural [B, T*H*W, heads, d] <-> tiled [B, heads, n_padded, d] (vsa_tile_permute)."""
    info = layout_info(lay)
    src_shape, dst_shape = _natural_shape(lay, info), _tiled_shape(lay, info)
    if inverse:
        src_shape, dst_shape = dst_shape, src_shape
    _want(src, "src", (torch.float32, torch.bfloat16), src_shape)
    if out is None:
        out = torch.empty(dst_shape, dtype=src.dtype, device=src.device)
    _want(out, "out", src.dtype, dst_shape)
    c = lay.c()
    check(lib().vsa_tile_permute(ctypes.byref(c), _DT.get(src.dtype, -1), _ptr(src), _ptr(out),
                                 1 if inverse else 0, _stream(stream)))
    return out


def tile_permute_v(lay: Layout, src: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """bf16 natural [B, T*H*W, heads, d] -> tiled V in the bf16 P.V operand
    layout [B, heads, n_padded, d] (vsa_tile_permute_v), for the forwards'
    ``v_operand=True``."""
    info = layout_info(lay)
    nat, tiled = _natural_shape(lay, info), _tiled_shape(lay, info)
    _want(src, "src", torch.bfloat16, nat)
    if out is None:
        out = torch.empty(tiled, dtype=torch.bfloat16, device=src.device)
    _want(out, "out", torch.bfloat16, tiled)
    c = lay.c()
    check(lib().vsa_tile_permute_v(ctypes.byref(c), _ptr(src), _ptr(out), _stream(stream)))
    return out


def tile_permute_pool(lay: Layout, src: torch.Tensor, out: Optional[torch.Tensor] = None,
                      pooled: Optional[torch.Tensor] = None, stream=None, means_only: bool = False):
    """bf16 natural -> tiled permute that also returns the fp32 tile means
    [B, heads, n_tiles, d] (vsa_tile_permute_pool): (tiled, pooled); with
    ``means_only`` no tiled copy is written: (None, pooled)."""
    info = layout_info(lay)
    _want(src, "src", torch.bfloat16, _natural_shape(lay, info))
    if out is None and not means_only:
        out = torch.empty(_tiled_shape(lay, info), dtype=src.dtype, device=src.device)
    if pooled is None:
        pooled = torch.empty((lay.batch, lay.heads, info.n_tiles, lay.head_dim),
                             dtype=torch.float32, device=src.device)
    if not means_only:
        _want(out, "out", torch.bfloat16, _tiled_shape(lay, info))
    else:
        out = None
    _want(pooled, "pooled", torch.float32, (lay.batch, lay.heads, info.n_tiles, lay.head_dim))
    c = lay.c()
    check(lib().vsa_tile_permute_pool(ctypes.byref(c), _ptr(src), _ptr(out), _ptr(pooled),
                                      _stream(stream)))
    return out, pooled


def build_mask_window(lay: Layout, radius: Tuple[int, int, int], max_kv: Optional[int] = None,
                      device="cuda", stream=None):
    """Head-invariant fixed lists (vsa_build_mask_window): (kv_idx [n_tiles, max_kv], kv_cnt)."""
    info = layout_info(lay)
    if max_kv is None:
        max_kv = info.n_tiles
    kv_idx = torch.empty((info.n_tiles, max_kv), dtype=torch.int32, device=device)
    kv_cnt = torch.empty((info.n_tiles,), dtype=torch.int32, device=device)
    c = lay.c()
    check(lib().vsa_build_mask_window(ctypes.byref(c), int(radius[0]), int(radius[1]),
                                      int(radius[2]), int(max_kv), _ptr(kv_idx), _ptr(kv_cnt),
                                      _stream(stream)))
    return kv_idx, kv_cnt


def build_mask_window_grouped(lay: Layout, group: Tuple[int, int, int],
                              extent: Tuple[int, int, int], max_kv: Optional[int] = None,
                              stream=None):
    """Big-tile window lists (vsa_build_mask_window_grouped): groups of `group`
    layout tiles, window extents counted in groups. Returns (kv_idx, kv_cnt)."""
    info = layout_info(lay)
    n = info.n_tiles
    if max_kv is None:
        grid = (info.tiles_t, info.tiles_h, info.tiles_w)
        max_kv = 1
        for m, g, e in zip(grid, group, extent):
            max_kv *= min(m, g * e)
    kv_idx = torch.empty((n, max_kv), dtype=torch.int32, device="cuda")
    kv_cnt = torch.empty((n,), dtype=torch.int32, device="cuda")
    c = lay.c()
    check(lib().vsa_build_mask_window_grouped(ctypes.byref(c), *(int(x) for x in group),
                                              *(int(x) for x in extent), int(max_kv),
                                              _ptr(kv_idx), _ptr(kv_cnt), _stream(stream)))
    return kv_idx, kv_cnt


def quant_fp8_tiles_grouped(lay: Layout, x_tiled: torch.Tensor, group: Tuple[int, int, int],
                            stream=None, v_operand: bool = False):
    """e4m3 codes with one scale per group of tiles (vsa_quant_fp8_tiles_grouped);
    the group's scale is stored for each of its tiles."""
    info = layout_info(lay)
    _want(x_tiled, "x_tiled", torch.bfloat16, _tiled_shape(lay, info))
    codes = torch.empty(x_tiled.shape, dtype=torch.uint8, device=x_tiled.device)
    scales = torch.empty((lay.batch, lay.heads, info.n_tiles), dtype=torch.float32,
                         device=x_tiled.device)
    c = lay.c()
    check(lib().vsa_quant_fp8_tiles_grouped(ctypes.byref(c), *(int(x) for x in group), _ptr(x_tiled),
                                            _ptr(codes), _ptr(scales), int(bool(v_operand)),
                                            _stream(stream)))
    return codes, scales


def topk_workspace_bytes(lay: Layout) -> int:
    c = lay.c()
    return int(lib().vsa_build_mask_topk_workspace(ctypes.byref(c)))


def build_mask_topk(lay: Layout, q_tiled: torch.Tensor, k_tiled: torch.Tensor,
                    coarse_scale: Optional[float] = None, top_k: int = 0, top_p: float = 0.0,
                    k_floor: int = 0, max_kv: Optional[int] = None, want_scores: bool = False,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """Routed lists per (b, head) (vsa_build_mask_topk): (kv_idx, kv_cnt, scores or None)."""
    info = layout_info(lay)
    n = info.n_tiles
    if coarse_scale is None:
        coarse_scale = 1.0 / math.sqrt(lay.head_dim)
    if max_kv is None:
        max_kv = n if top_p > 0 else min(top_k, n)
    dev = q_tiled.device
    _want(q_tiled, "q_tiled", torch.bfloat16, _tiled_shape(lay, info))
    _want(k_tiled, "k_tiled", torch.bfloat16, _tiled_shape(lay, info))
    kv_idx = torch.empty((lay.batch, lay.heads, n, max_kv), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty((lay.batch, lay.heads, n), dtype=torch.int32, device=dev)
    scores = torch.empty((lay.batch, lay.heads, n, n), dtype=torch.float32, device=dev) \
        if want_scores else None
    need = topk_workspace_bytes(lay)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    c = lay.c()
    check(lib().vsa_build_mask_topk(ctypes.byref(c), _ptr(q_tiled), _ptr(k_tiled),
                                    float(coarse_scale), int(top_k), float(top_p), int(k_floor),
                                    int(max_kv), _ptr(kv_idx), _ptr(kv_cnt), _ptr(scores),
                                    _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
    return kv_idx, kv_cnt, scores


def build_mask_topk_pooled(lay: Layout, q_pooled: torch.Tensor, k_pooled: torch.Tensor,
                           coarse_scale: Optional[float] = None, top_k: int = 0,
                           top_p: float = 0.0, k_floor: int = 0, max_kv: Optional[int] = None,
                           want_scores: bool = False, workspace: Optional[torch.Tensor] = None,
                           stream=None):
    """Routed lists from pooled tile means (vsa_build_mask_topk_pooled):
    (kv_idx, kv_cnt, scores or None), as build_mask_topk. Needs no workspace
    (``workspace`` is accepted and ignored)."""
    info = layout_info(lay)
    n = info.n_tiles
    if coarse_scale is None:
        coarse_scale = 1.0 / math.sqrt(lay.head_dim)
    if max_kv is None:
        max_kv = n if top_p > 0 else min(top_k, n)
    dev = q_pooled.device
    for t in (q_pooled, k_pooled):
        if t.dtype != torch.float32 or tuple(t.shape) != (lay.batch, lay.heads, n, lay.head_dim):
            raise ValueError("pooled means must be float32 [B, heads, n_tiles, d]")
    kv_idx = torch.empty((lay.batch, lay.heads, n, max_kv), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty((lay.batch, lay.heads, n), dtype=torch.int32, device=dev)
    scores = torch.empty((lay.batch, lay.heads, n, n), dtype=torch.float32, device=dev) \
        if want_scores else None
    c = lay.c()
    check(lib().vsa_build_mask_topk_pooled(ctypes.byref(c), _ptr(q_pooled), _ptr(k_pooled),
                                           float(coarse_scale), int(top_k), float(top_p),
                                           int(k_floor), int(max_kv), _ptr(kv_idx), _ptr(kv_cnt),
                                           _ptr(scores), _ptr(workspace),
                                           0 if workspace is None else _ws_bytes(workspace),
                                           _stream(stream)))
    return kv_idx, kv_cnt, scores


def build_work_order(lay: Layout, kv_cnt: torch.Tensor, stream=None) -> torch.Tensor:
    """Heavy-first dealing order of the routed walks (vsa_build_work_order):
    int32 [B * heads * n_tiles], heads by total pairs then query tiles by list
    length, both descending, ties in index order."""
    info = layout_info(lay)
    _want(kv_cnt, "kv_cnt", torch.int32, (lay.batch, lay.heads, info.n_tiles))
    order = torch.empty(lay.batch * lay.heads * info.n_tiles, dtype=torch.int32, device=kv_cnt.device)
    c = lay.c()
    check(lib().vsa_build_work_order(ctypes.byref(c), _ptr(kv_cnt), _ptr(order), _stream(stream)))
    return order


def _check_order(lay: Layout, info, kv_idx, work_order) -> None:
    if work_order is None:
        return
    if kv_idx is None or kv_idx.dim() != 4:
        raise ValueError("work_order applies to per-head [B, heads, n_tiles, max_kv] lists only")
    _want(work_order, "work_order", torch.int32, (lay.batch * lay.heads * info.n_tiles,))


def quant_fp8_tiles(lay: Layout, x_tiled: torch.Tensor, stream=None, v_operand: bool = False):
    """Per-tile e4m3 codes (uint8, same shape) and scales [B, heads, n_tiles].

    vsa_quant_fp8_tiles, or with ``v_operand`` vsa_quant_fp8_tiles_v (each
    tile's codes channel-major in the fp8 P.V operand order, for V).
    """
    info = layout_info(lay)
    _want(x_tiled, "x_tiled", torch.bfloat16, _tiled_shape(lay, info))
    codes = torch.empty(x_tiled.shape, dtype=torch.uint8, device=x_tiled.device)
    scales = torch.empty((lay.batch, lay.heads, info.n_tiles), dtype=torch.float32,
                         device=x_tiled.device)
    c = lay.c()
    fn = lib().vsa_quant_fp8_tiles_v if v_operand else lib().vsa_quant_fp8_tiles
    check(fn(ctypes.byref(c), _ptr(x_tiled), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def quant_fp8_tiles_nat(lay: Layout, x_nat: torch.Tensor, v_operand: bool = False,
                        want_pooled: bool = False, stream=None):
    """Natural-order bf16 [B, T*H*W, heads, d] -> tiled e4m3 codes and scales in
    one pass (vsa_quant_fp8_tiles_nat); the same bits as tile_permute then
    quant_fp8_tiles. Returns (codes, scales, pooled means or None)."""
    info = layout_info(lay)
    _want(x_nat, "x_nat", torch.bfloat16, _natural_shape(lay, info))
    dev = x_nat.device
    codes = torch.empty(_tiled_shape(lay, info), dtype=torch.uint8, device=dev)
    scales = torch.empty((lay.batch, lay.heads, info.n_tiles), dtype=torch.float32, device=dev)
    pooled = torch.empty((lay.batch, lay.heads, info.n_tiles, lay.head_dim), dtype=torch.float32,
                         device=dev) if want_pooled else None
    c = lay.c()
    check(lib().vsa_quant_fp8_tiles_nat(ctypes.byref(c), _ptr(x_nat), _ptr(codes), _ptr(scales),
                                        _ptr(pooled), int(bool(v_operand)), _stream(stream)))
    return codes, scales, pooled


def block_sparse_attn_fwd_fp8_nat(lay: Layout, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  scales: Tuple[torch.Tensor, torch.Tensor, torch.Tensor],
                                  kv_idx: Optional[torch.Tensor] = None,
                                  kv_cnt: Optional[torch.Tensor] = None,
                                  softmax_scale: Optional[float] = None, want_lse: bool = False,
                                  out: Optional[torch.Tensor] = None,
                                  lse: Optional[torch.Tensor] = None, stream=None,
                                  v_operand: bool = False, per_tile_walk: bool = False,
                                  work_order: Optional[torch.Tensor] = None):
    """fp8 forward with O written in the natural order [B, T*H*W, heads, d]
    (vsa_block_sparse_attn_fwd_fp8_nat); q/k/v tiled e4m3 codes. Returns
    (out, lse or None); lse tiled. ``work_order``: from build_work_order
    (per-head lists only)."""
    info = layout_info(lay)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(lay.head_dim)
    tiled = _tiled_shape(lay, info)
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _want(t, nm, torch.uint8, tiled)
    for nm, t in zip(("q_scale", "k_scale", "v_scale"), scales):
        _want(t, nm, torch.float32, (lay.batch, lay.heads, info.n_tiles))
    _check_lists(lay, info, kv_idx, kv_cnt)
    if per_tile_walk and kv_idx is not None and kv_idx.dim() != 2:
        raise ValueError("per_tile_walk applies to a shared [n_tiles, max_kv] table only")
    _check_order(lay, info, kv_idx, work_order)
    if out is None:
        out = torch.empty(_natural_shape(lay, info), dtype=torch.bfloat16, device=q.device)
    _want(out, "out", torch.bfloat16, _natural_shape(lay, info))
    if want_lse and lse is None:
        lse = torch.empty((lay.batch, lay.heads, info.n_padded), dtype=torch.float32, device=q.device)
    if lse is not None:
        _want(lse, "lse", torch.float32, (lay.batch, lay.heads, info.n_padded))
    if kv_idx is not None:
        max_kv = kv_idx.shape[-1]
        list_mode = (2 if per_tile_walk else 0) if kv_idx.dim() == 2 else 1
    else:
        max_kv, list_mode = 0, 0
    qs, ks, vs = scales
    c = lay.c()
    check(lib().vsa_block_sparse_attn_fwd_fp8_nat(
        ctypes.byref(c), VSA_FP8_E4M3_VOP if v_operand else VSA_FP8_E4M3, _ptr(q), _ptr(k), _ptr(v),
        _ptr(qs), _ptr(ks), _ptr(vs), _ptr(kv_idx), _ptr(kv_cnt), int(max_kv), list_mode,
        _ptr(work_order), float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def block_sparse_attn_fwd(lay: Layout, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          kv_idx: Optional[torch.Tensor] = None,
                          kv_cnt: Optional[torch.Tensor] = None,
                          softmax_scale: Optional[float] = None,
                          scales: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                          want_lse: bool = False, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, stream=None, v_operand: bool = False,
                          per_tile_walk: bool = False, work_order: Optional[torch.Tensor] = None):
    """Block-sparse attention forward (vsa_block_sparse_attn_fwd).

    q/k/v tiled; float32 -> float32 out, bfloat16 -> bfloat16 out, uint8 e4m3
    codes (with ``scales`` = (q_scale, k_scale, v_scale)) -> bfloat16 out;
    ``v_operand``: v holds codes from quant_fp8_tiles(..., v_operand=True),
    or (bf16) the output of tile_permute_v.
    kv_idx 2-D [n_tiles, max_kv] = one shared table; 4-D [B, heads, n_tiles,
    max_kv] = per-(b, head) lists; None = dense. ``per_tile_walk`` (2-D
    tables only): each query tile walks its own list (list_mode 2).
    ``work_order`` (per-head lists only): the dealing order from
    build_work_order; the output is the same with or without it.
    Returns (out, lse or None).
    """
    info = layout_info(lay)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(lay.head_dim)
    tiled = _tiled_shape(lay, info)
    _want(q, "q", (torch.float32, torch.bfloat16, torch.uint8), tiled)
    _want(k, "k", q.dtype, tiled)
    _want(v, "v", q.dtype, tiled)
    _check_lists(lay, info, kv_idx, kv_cnt)
    if per_tile_walk and kv_idx is not None and kv_idx.dim() != 2:
        raise ValueError("per_tile_walk applies to a shared [n_tiles, max_kv] table only")
    _check_order(lay, info, kv_idx, work_order)
    if q.dtype == torch.uint8:
        dtype, odt = VSA_FP8_E4M3, torch.bfloat16
        if scales is None:
            raise ValueError("fp8 codes need (q_scale, k_scale, v_scale)")
        for nm, t in zip(("q_scale", "k_scale", "v_scale"), scales):
            _want(t, nm, torch.float32, (lay.batch, lay.heads, info.n_tiles))
        if v_operand:
            dtype = VSA_FP8_E4M3_VOP
    elif scales is not None:
        raise ValueError("scales apply to fp8 codes only")
    elif v_operand:
        if q.dtype != torch.bfloat16:
            raise ValueError("v_operand applies to bf16 tensors or fp8 codes")
        dtype, odt = VSA_BF16_VOP, q.dtype
    else:
        dtype, odt = _DT.get(q.dtype, -1), q.dtype
    if out is None:
        out = torch.empty(tiled, dtype=odt, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((lay.batch, lay.heads, info.n_padded), dtype=torch.float32,
                          device=q.device)
    _want(out, "out", odt, tiled)
    if lse is not None:
        _want(lse, "lse", torch.float32, (lay.batch, lay.heads, info.n_padded))
    if kv_idx is not None:
        max_kv = kv_idx.shape[-1]
        list_mode = (2 if per_tile_walk else 0) if kv_idx.dim() == 2 else 1
    else:
        max_kv, list_mode = 0, 0
    qs, ks, vs = scales if scales is not None else (None, None, None)
    c = lay.c()
    check(lib().vsa_block_sparse_attn_fwd(
        ctypes.byref(c), dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(qs), _ptr(ks), _ptr(vs),
        _ptr(kv_idx), _ptr(kv_cnt), int(max_kv), list_mode, _ptr(work_order), float(softmax_scale),
        _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def build_transposed_lists(lay: Layout, kv_idx: torch.Tensor, kv_cnt: torch.Tensor, stream=None):
    """Per key tile, the ascending query tiles whose list holds it
    (vsa_build_transposed_lists): (q_idx, q_cnt), 2-D / 1-D for a shared table,
    4-D / 3-D for per-(b, head) lists."""
    info = layout_info(lay)
    n = info.n_tiles
    _check_lists(lay, info, kv_idx, kv_cnt)
    list_mode = 0 if kv_idx.dim() == 2 else 1
    lead = () if list_mode == 0 else (lay.batch, lay.heads)
    q_idx = torch.empty(lead + (n, n), dtype=torch.int32, device=kv_idx.device)
    q_cnt = torch.empty(lead + (n,), dtype=torch.int32, device=kv_idx.device)
    c = lay.c()
    check(lib().vsa_build_transposed_lists(ctypes.byref(c), _ptr(kv_idx), _ptr(kv_cnt),
                                           int(kv_idx.shape[-1]), list_mode, _ptr(q_idx),
                                           _ptr(q_cnt), _stream(stream)))
    return q_idx, q_cnt


def bwd_workspace_bytes(lay: Layout) -> int:
    c = lay.c()
    return int(lib().vsa_block_sparse_attn_bwd_workspace(ctypes.byref(c)))


def block_sparse_attn_bwd(lay: Layout, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                          kv_idx: Optional[torch.Tensor] = None,
                          kv_cnt: Optional[torch.Tensor] = None,
                          q_idx: Optional[torch.Tensor] = None,
                          q_cnt: Optional[torch.Tensor] = None,
                          softmax_scale: Optional[float] = None,
                          grads: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dq, dk, dv) of block_sparse_attn_fwd (vsa_block_sparse_attn_bwd).

    Same tensors, lists and scale as the forward call, plus its output and
    lse and the upstream gradient ``dout``. The transposed lists are built
    here when kv_idx is given and q_idx is not.
    """
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(lay.head_dim)
    info = layout_info(lay)
    tiled = _tiled_shape(lay, info)
    _want(q, "q", (torch.float32, torch.bfloat16), tiled)
    for nm, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _want(t, nm, q.dtype, tiled)
    _want(lse, "lse", torch.float32, (lay.batch, lay.heads, info.n_padded))
    _check_lists(lay, info, kv_idx, kv_cnt)
    if q_idx is not None or q_cnt is not None:
        if kv_idx is None:
            raise ValueError("q_idx / q_cnt need the forward lists kv_idx / kv_cnt")
        n = int(info.n_tiles)
        lead = (n,) if kv_idx.dim() == 2 else (lay.batch, lay.heads, n)
        _want(q_idx, "q_idx", torch.int32, lead + (n,))
        _want(q_cnt, "q_cnt", torch.int32, lead)
    dtype = _DT.get(q.dtype, -1)
    if kv_idx is not None and q_idx is None:
        q_idx, q_cnt = build_transposed_lists(lay, kv_idx, kv_cnt, stream=stream)
    if kv_idx is not None:
        max_kv = kv_idx.shape[-1]
        list_mode = 0 if kv_idx.dim() == 2 else 1
    else:
        max_kv, list_mode = 0, 0
    if grads is None:
        grads = tuple(torch.empty_like(x) for x in (q, k, v))
    dq, dk, dv = grads
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _want(t, nm, q.dtype, tiled)
    need = bwd_workspace_bytes(lay)
    if workspace is None:
        workspace = torch.empty((max(need, 8),), dtype=torch.uint8, device=q.device)
    c = lay.c()
    check(lib().vsa_block_sparse_attn_bwd(
        ctypes.byref(c), dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
        _ptr(kv_idx), _ptr(kv_cnt), int(max_kv), _ptr(q_idx), _ptr(q_cnt), list_mode,
        float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), _ws_bytes(workspace),
        _stream(stream)))
    return dq, dk, dv


def block_sparse_attn_bwd_noalloc(lay: Layout, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                                  kv_idx: Optional[torch.Tensor] = None,
                                  kv_cnt: Optional[torch.Tensor] = None,
                                  q_idx: Optional[torch.Tensor] = None,
                                  q_cnt: Optional[torch.Tensor] = None,
                                  softmax_scale: Optional[float] = None,
                                  grads: Tuple[torch.Tensor, torch.Tensor, torch.Tensor] = None,
                                  stream=None):
    """block_sparse_attn_bwd without a workspace (vsa_block_sparse_attn_bwd_noalloc):
    the library's built-in scratch holds the row statistics. ``grads`` (dq, dk,
    dv) and, for listed attention, the transposed lists must be passed in, so
    the call allocates nothing."""
    if grads is None:
        raise ValueError("grads (dq, dk, dv) must be given: this call allocates nothing")
    if kv_idx is not None and q_idx is None:
        raise ValueError("q_idx / q_cnt must be given: this call allocates nothing")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(lay.head_dim)
    info = layout_info(lay)
    tiled = _tiled_shape(lay, info)
    _want(q, "q", (torch.float32, torch.bfloat16), tiled)
    for nm, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _want(t, nm, q.dtype, tiled)
    _want(lse, "lse", torch.float32, (lay.batch, lay.heads, info.n_padded))
    _check_lists(lay, info, kv_idx, kv_cnt)
    if kv_idx is not None:
        n = int(info.n_tiles)
        lead = (n,) if kv_idx.dim() == 2 else (lay.batch, lay.heads, n)
        _want(q_idx, "q_idx", torch.int32, lead + (n,))
        _want(q_cnt, "q_cnt", torch.int32, lead)
        max_kv, list_mode = kv_idx.shape[-1], (0 if kv_idx.dim() == 2 else 1)
    else:
        max_kv, list_mode = 0, 0
    dq, dk, dv = grads
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _want(t, nm, q.dtype, tiled)
    c = lay.c()
    check(lib().vsa_block_sparse_attn_bwd_noalloc(
        ctypes.byref(c), _DT.get(q.dtype, -1), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
        _ptr(lse), _ptr(kv_idx), _ptr(kv_cnt), int(max_kv), _ptr(q_idx), _ptr(q_cnt), list_mode,
        float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))
    return dq, dk, dv


def block_sparse_attn_fwd_nat(lay: Layout, q_nat: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              kv_idx: Optional[torch.Tensor] = None,
                              kv_cnt: Optional[torch.Tensor] = None,
                              softmax_scale: Optional[float] = None, want_lse: bool = False,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              stream=None, per_tile_walk: bool = False,
                              work_order: Optional[torch.Tensor] = None, v_operand: bool = False):
    """Forward with natural-order Q in and O out (vsa_block_sparse_attn_fwd_nat):
    q_nat and the returned out are [B, T*H*W, heads, d]; k and v tiled
    (``v_operand``: bf16 v from tile_permute_v).
    Returns (out, lse or None); lse in the tiled order."""
    info = layout_info(lay)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(lay.head_dim)
    nat, tiled = _natural_shape(lay, info), _tiled_shape(lay, info)
    _want(q_nat, "q_nat", (torch.float32, torch.bfloat16), nat)
    _want(k, "k", q_nat.dtype, tiled)
    _want(v, "v", q_nat.dtype, tiled)
    _check_lists(lay, info, kv_idx, kv_cnt)
    if per_tile_walk and kv_idx is not None and kv_idx.dim() != 2:
        raise ValueError("per_tile_walk applies to a shared [n_tiles, max_kv] table only")
    _check_order(lay, info, kv_idx, work_order)
    dtype = _DT.get(q_nat.dtype, -1)
    if v_operand:
        if q_nat.dtype != torch.bfloat16:
            raise ValueError("v_operand applies to bf16 tensors")
        dtype = VSA_BF16_VOP
    if out is None:
        out = torch.empty_like(q_nat)
    if want_lse and lse is None:
        lse = torch.empty((lay.batch, lay.heads, info.n_padded), dtype=torch.float32,
                          device=q_nat.device)
    _want(out, "out", q_nat.dtype, nat)
    if lse is not None:
        _want(lse, "lse", torch.float32, (lay.batch, lay.heads, info.n_padded))
    if kv_idx is not None:
        max_kv = kv_idx.shape[-1]
        list_mode = (2 if per_tile_walk else 0) if kv_idx.dim() == 2 else 1
    else:
        max_kv, list_mode = 0, 0
    c = lay.c()
    check(lib().vsa_block_sparse_attn_fwd_nat(
        ctypes.byref(c), dtype, _ptr(q_nat), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt),
        int(max_kv), list_mode, _ptr(work_order), float(softmax_scale), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out, lse
