"""Helpers shared by the GPU parity tests (inputs, layouts, comparisons)."""
import functools
import sys

import numpy as np
import torch

from oracle.layout import Layout as OLayout
from synth import CONFIGS, bf16_bits, make_qkv

DEV = "cuda"


def announce(msg: str) -> None:
    print(f"[gpu-step] {msg}", file=sys.__stderr__, flush=True)


@functools.lru_cache(maxsize=None)
def inputs(name):
    """Natural-order float32 (q, k, v) of a workload, cached per session."""
    return make_qkv(CONFIGS[name])


def layouts(cfg, heads=None):
    import block_sparse_attention_token_amd as vsa
    h = heads or cfg.heads
    o = OLayout(T=cfg.T, H=cfg.H, W=cfg.W, heads=h, head_dim=cfg.head_dim, kind=cfg.kind,
                tile=cfg.tile, stride=cfg.stride)
    b = vsa.Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=h, head_dim=cfg.head_dim, kind=cfg.kind,
                   tile=cfg.tile, stride=cfg.stride)
    return o, b


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


def ref_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x).view(np.int16)
    return np.ascontiguousarray(x, dtype=np.float32).view(np.int32)


def errors(gpu: np.ndarray, ref: np.ndarray):
    err = gpu.astype(np.float64) - ref
    return float(np.abs(err).max()), float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))


def lists_to_device(idx: np.ndarray, cnt: np.ndarray):
    """Oracle lists (-1 padded) -> int32 device tensors; unused slots set to 0."""
    i = np.where(idx < 0, 0, idx).astype(np.int32)
    return torch.from_numpy(np.ascontiguousarray(i)).to(DEV), \
        torch.from_numpy(np.ascontiguousarray(cnt.astype(np.int32))).to(DEV)


def table_from_lists(lists, width=None):
    """Head-invariant list-of-lists -> (-1 padded array [n, width], counts)."""
    n = len(lists)
    width = width or max(1, max(len(x) for x in lists))
    idx = np.full((n, width), -1, dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    for i, row in enumerate(lists):
        idx[i, :len(row)] = row
        cnt[i] = len(row)
    return idx, cnt
