"""ctypes loader and declarations for libvsa.so (see include/vsa.h).

The library must already be built in-tree (``python -m
block_sparse_attention_token_amd.build``); importing fails loudly otherwise.
torch is imported first so that libvsa binds to the HIP runtime torch uses.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libvsa links against)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvsa.so")

VSA_OK = 0
VSA_ERR_INVALID = 1
VSA_ERR_UNSUPPORTED = 2
VSA_ERR_WORKSPACE = 3
VSA_ERR_HIP = 4

VSA_F32 = 0
VSA_BF16 = 1
VSA_FP8_E4M3 = 2
VSA_FP8_E4M3_VOP = 3
VSA_BF16_VOP = 4

VSA_TILE3D = 0
VSA_SKIPARSE2D = 1

EXPORTED = (
    "vsa_layout_query", "vsa_tile_permute", "vsa_tile_permute_v", "vsa_build_mask_window",
    "vsa_build_mask_topk",
    "vsa_build_mask_topk_workspace", "vsa_quant_fp8_tiles", "vsa_quant_fp8_tiles_v",
    "vsa_block_sparse_attn_fwd", "vsa_block_sparse_attn_fwd_nat", "vsa_build_mask_window_grouped",
    "vsa_quant_fp8_tiles_grouped", "vsa_tile_permute_pool", "vsa_build_mask_topk_pooled",
    "vsa_build_transposed_lists", "vsa_block_sparse_attn_bwd_workspace",
    "vsa_block_sparse_attn_bwd", "vsa_block_sparse_attn_bwd_noalloc", "vsa_quant_fp8_tiles_nat",
    "vsa_block_sparse_attn_fwd_fp8_nat", "vsa_build_work_order", "vsa_status_string",
    "vsa_last_error", "vsa_version",
)


class VsaLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "head_dim", "T", "H", "W", "kind",
        "tile_t", "tile_h", "tile_w", "stride_h", "stride_w")]


class VsaLayoutInfo(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_padded", ctypes.c_int64)] + \
        [(n, ctypes.c_int32) for n in ("n_tiles", "tile_tokens", "n_groups", "tiles_per_group",
                                       "group_len", "tiles_t", "tiles_h", "tiles_w")]


class VsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {0: "VSA_OK", 1: "VSA_ERR_INVALID", 2: "VSA_ERR_UNSUPPORTED", 3: "VSA_ERR_WORKSPACE",
           4: "VSA_ERR_HIP"}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libvsa; raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_token_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    LP = ctypes.POINTER(VsaLayout)
    L.vsa_layout_query.argtypes = [LP, ctypes.POINTER(VsaLayoutInfo)]
    L.vsa_tile_permute.argtypes = [LP, I32, P, P, I32, P]
    L.vsa_tile_permute_v.argtypes = [LP, P, P, P]
    L.vsa_build_mask_window.argtypes = [LP, I32, I32, I32, I32, P, P, P]
    L.vsa_build_mask_topk.argtypes = [LP, P, P, F32, I32, F32, I32, I32, P, P, P, P, SZ, P]
    L.vsa_build_mask_topk_workspace.argtypes = [LP]
    L.vsa_build_mask_topk_workspace.restype = SZ
    L.vsa_quant_fp8_tiles.argtypes = [LP, P, P, P, P]
    L.vsa_quant_fp8_tiles_v.argtypes = [LP, P, P, P, P]
    L.vsa_block_sparse_attn_fwd.argtypes = [LP, I32, P, P, P, P, P, P, P, P, I32, I32, P, F32, P, P, P]
    L.vsa_block_sparse_attn_fwd_nat.argtypes = [LP, I32, P, P, P, P, P, I32, I32, P, F32, P, P, P]
    L.vsa_build_work_order.argtypes = [LP, P, P, P]
    L.vsa_build_mask_window_grouped.argtypes = [LP, I32, I32, I32, I32, I32, I32, I32, P, P, P]
    L.vsa_quant_fp8_tiles_grouped.argtypes = [LP, I32, I32, I32, P, P, P, I32, P]
    L.vsa_build_transposed_lists.argtypes = [LP, P, P, I32, I32, P, P, P]
    L.vsa_block_sparse_attn_bwd_workspace.argtypes = [LP]
    L.vsa_block_sparse_attn_bwd_workspace.restype = SZ
    L.vsa_block_sparse_attn_bwd.argtypes = [LP, I32, P, P, P, P, P, P, P, P, I32, P, P, I32, F32,
                                            P, P, P, P, SZ, P]
    L.vsa_block_sparse_attn_bwd_noalloc.argtypes = [LP, I32, P, P, P, P, P, P, P, P, I32, P, P, I32,
                                                    F32, P, P, P, P]
    L.vsa_tile_permute_pool.argtypes = [LP, P, P, P, P]
    L.vsa_quant_fp8_tiles_nat.argtypes = [LP, P, P, P, P, I32, P]
    L.vsa_block_sparse_attn_fwd_fp8_nat.argtypes = [LP, I32, P, P, P, P, P, P, P, P, I32, I32, P, F32,
                                                    P, P, P]
    L.vsa_build_mask_topk_pooled.argtypes = [LP, P, P, F32, I32, F32, I32, I32, P, P, P, P, SZ, P]
    for name in ("vsa_layout_query", "vsa_tile_permute", "vsa_tile_permute_v", "vsa_build_mask_window",
                 "vsa_build_mask_topk", "vsa_quant_fp8_tiles", "vsa_quant_fp8_tiles_v",
                 "vsa_block_sparse_attn_fwd", "vsa_block_sparse_attn_fwd_nat",
                 "vsa_build_mask_window_grouped", "vsa_quant_fp8_tiles_grouped",
                 "vsa_tile_permute_pool", "vsa_build_mask_topk_pooled",
                 "vsa_build_transposed_lists", "vsa_block_sparse_attn_bwd",
                 "vsa_block_sparse_attn_bwd_noalloc", "vsa_quant_fp8_tiles_nat",
                 "vsa_block_sparse_attn_fwd_fp8_nat", "vsa_build_work_order"):
        getattr(L, name).restype = I32
    L.vsa_status_string.argtypes = [I32]
    L.vsa_status_string.restype = ctypes.c_char_p
    L.vsa_last_error.argtypes = []
    L.vsa_last_error.restype = ctypes.c_char_p
    L.vsa_version.argtypes = []
    L.vsa_version.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int) -> None:
    if status != VSA_OK:
        raise VsaError(status, lib().vsa_last_error().decode())
