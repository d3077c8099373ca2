"""GPU parity: tile permutation and fixed masks are bit-exact against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import layout as OL
from oracle import masks as OM
from oracle.layout import Layout as OLayout
from synth import CONFIGS, round_to_bf16
from tests.conftest import read_golden
from tests.gpu_util import (announce, host_bits, inputs, layouts, ref_bits, table_from_lists,
                            to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(CONFIGS))
def test_permute_roundtrip_bitexact(name):
    cfg = CONFIGS[name]
    olay, blay = layouts(cfg)
    q, k, v = inputs(name)
    x = k if name == "skiparse_768p" else q
    announce(f"permute {name} {x.shape}")
    xd = to_device(x, cfg.dtype)
    xt = vsa.tile_permute(blay, xd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(xt), ref_bits(OL.permute(x, olay), cfg.dtype))
    back = vsa.tile_permute(blay, xt, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(host_and_view(back), host_and_view(xd))


def host_and_view(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("grid,tile,kind,stride", [
    ((3, 5, 6), (2, 4, 4), "tile3d", (1, 1)),
    ((5, 7, 9), (4, 4, 4), "tile3d", (1, 1)),
    ((3, 4, 6), (1, 4, 4), "skiparse2d", (2, 2)),
    ((2, 6, 9), (1, 4, 8), "skiparse2d", (3, 3)),
    ((1, 1, 1), (4, 4, 4), "tile3d", (1, 1)),
])
def test_permute_small_grids_bitexact(grid, tile, kind, stride):
    T, H, W = grid
    olay = OLayout(T=T, H=H, W=W, heads=3, head_dim=8, kind=kind, tile=tile, stride=stride, batch=2)
    blay = vsa.Layout(T=T, H=H, W=W, heads=3, head_dim=8, kind=kind, tile=tile, stride=stride, batch=2)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, T * H * W, 3, 8)).astype(np.float32)
    announce(f"permute small {grid} {tile} {kind}")
    for dt in ("f32", "bf16"):
        xr = round_to_bf16(x) if dt == "bf16" else x
        xd = to_device(xr, dt)
        # canary-filled output proves the pad rows are written as zeros
        info = vsa.layout_info(blay)
        out = torch.full((2, 3, info.n_padded, 8), 7.0, dtype=xd.dtype, device="cuda")
        vsa.tile_permute(blay, xd, out=out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), ref_bits(OL.permute(xr, olay), dt))
        back = vsa.tile_permute(blay, out, inverse=True)
        torch.cuda.synchronize()
        assert torch.equal(host_and_view(back), host_and_view(xd))


def _check_lists(kv_idx, kv_cnt, lists):
    idx = kv_idx.cpu().numpy()
    cnt = kv_cnt.cpu().numpy()
    assert cnt.tolist() == [len(r) for r in lists]
    for i, row in enumerate(lists):
        assert idx[i, :len(row)].tolist() == row


@pytest.mark.parametrize("line", read_golden("window_masks.txt"))
def test_golden_window_masks(line):
    spec, _ = line.split(":")
    T, H, W, tt, th, tw, rt, rh, rw = map(int, spec.split())
    olay = OLayout(T=T, H=H, W=W, heads=1, head_dim=8, tile=(tt, th, tw))
    blay = vsa.Layout(T=T, H=H, W=W, heads=1, head_dim=8, tile=(tt, th, tw))
    announce(f"mask window {spec}")
    kv_idx, kv_cnt = vsa.build_mask_window(blay, (rt, rh, rw))
    torch.cuda.synchronize()
    _check_lists(kv_idx, kv_cnt, OM.window_lists(olay, rt, rh, rw))


@pytest.mark.parametrize("name,radius", [("tiny_window_f32", (1, 1, 1)), ("window_480p", (1, 2, 2)),
                                         ("skiparse_768p", (0, 0, 0)), ("window_480p", (-1, 0, 0)),
                                         ("fp8_topp_720p", (1, 1, 1))])
def test_workload_masks_bitexact(name, radius):
    cfg = CONFIGS[name]
    olay, blay = layouts(cfg)
    announce(f"mask {name} {radius}")
    lists = OM.window_lists(olay, *radius)
    width = max(len(r) for r in lists)
    kv_idx, kv_cnt = vsa.build_mask_window(blay, radius, max_kv=width)
    torch.cuda.synchronize()
    _check_lists(kv_idx, kv_cnt, lists)
    # run-to-run determinism
    kv_idx2, kv_cnt2 = vsa.build_mask_window(blay, radius, max_kv=width)
    torch.cuda.synchronize()
    assert torch.equal(kv_cnt, kv_cnt2)
    cnt = kv_cnt.cpu().numpy()
    a, b = kv_idx.cpu().numpy(), kv_idx2.cpu().numpy()
    for i, c in enumerate(cnt):
        assert np.array_equal(a[i, :c], b[i, :c])


def test_mask_max_kv_too_small_writes_nothing():
    cfg = CONFIGS["window_480p"]
    _, blay = layouts(cfg)
    kv_idx = torch.full((624, 74), -5, dtype=torch.int32, device="cuda")
    kv_cnt = torch.full((624,), -5, dtype=torch.int32, device="cuda")
    c = blay.c()
    st = vsa._lib.lib().vsa_build_mask_window(ctypes.byref(c), 1, 2, 2, 74,
                                              ctypes.c_void_p(kv_idx.data_ptr()),
                                              ctypes.c_void_p(kv_cnt.data_ptr()), None)
    assert st == vsa._lib.VSA_ERR_INVALID
    torch.cuda.synchronize()
    assert bool((kv_idx == -5).all()) and bool((kv_cnt == -5).all())
