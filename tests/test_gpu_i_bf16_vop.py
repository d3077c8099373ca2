"""bf16 V in the P.V operand layout (vsa_tile_permute_v, dtype VSA_BF16_VOP).

The layout is a storage order of V only (FVAttn summary: video-aware block
organisation); the attention it feeds is the forward's (OSP-Next wiki TL;DR:
FlashAttention-compatible sparse attention).

* vsa_tile_permute_v against the oracle's tile permute followed by its bf16
  P.V operand layout, bit for bit (pure data movement), on ragged 3D grids
  and a Skiparse grid, head_dim 64, 128 and 256, pad tokens zero;
* every bf16 forward with ``v_operand`` gives the same bits as with
  token-major V: dense, shared windows (grouped and per-tile walks), routed
  per-head lists with and without a work order, tiled and natural-order Q/O,
  head_dim 64 and 128, 3D tiles and Skiparse groups with a padded last tile; at full size the 768p Skiparse layer, the 480p
  window layer (both walks) and the routed top-32 layer.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import layout as OL
from synth import CONFIGS, bf16_bits, round_to_bf16
from tests.gpu_util import announce, inputs, layouts, lists_to_device, to_device
from tests.test_gpu_h_work_order import _routed_lists

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("grid,heads,d,kind,stride", [
    ((9, 14, 22), 3, 128, "tile3d", (2, 2)),
    ((5, 9, 7), 2, 64, "tile3d", (2, 2)),
    ((3, 6, 10), 1, 256, "tile3d", (2, 2)),
    ((4, 8, 12), 2, 128, "skiparse2d", (2, 2)),
])
def test_permute_v_matches_oracle_layout(grid, heads, d, kind, stride):
    _gpu()
    T, H, W = grid
    B = 2
    announce(f"permute_v: grid={grid} heads={heads} d={d} kind={kind}")
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind=kind, tile=(4, 4, 4), stride=stride)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind=kind, tile=(4, 4, 4), stride=stride,
                      batch=B)
    rng = np.random.default_rng(41)
    x = rng.standard_normal((B, olay.n_tokens, heads, d)).astype(np.float32)
    bits = bf16_bits(x).view(np.int16)
    got = vsa.tile_permute_v(blay, to_device(x, "bf16"))
    torch.cuda.synchronize()
    want = OL.v_operand_layout_bf16(OL.permute(bits, olay), olay)
    assert np.array_equal(got.view(torch.int16).cpu().numpy(), want)


@pytest.mark.parametrize("d,kind,grid", [(128, "tile3d", (9, 14, 22)), (64, "tile3d", (9, 14, 22)),
                                          (128, "skiparse2d", (3, 12, 20))])
def test_forwards_identical_with_v_operand(d, kind, grid):
    _gpu()
    B, heads = 2, 3
    T, H, W = grid
    lay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind=kind, batch=B)
    info = vsa.layout_info(lay)
    n = info.n_tiles
    announce(f"bf16 V operand: forwards d={d} kind={kind} grid={grid}")
    rng = np.random.default_rng(42)
    x = [round_to_bf16(rng.standard_normal((B, info.n_tokens, heads, d)).astype(np.float32))
         for _ in range(3)]
    nat = [to_device(a, "bf16") for a in x]
    tq, tk, tv = (vsa.tile_permute(lay, a) for a in nat)
    vo = vsa.tile_permute_v(lay, nat[2])
    widx, wcnt = vsa.build_mask_window(lay, (1, 1, 1))
    ridx, rcnt = lists_to_device(*_routed_lists(rng, B, heads, n))
    order = vsa.build_work_order(lay, rcnt)
    cases = [("dense", dict()),
             ("window grouped", dict(kv_idx=widx, kv_cnt=wcnt)),
             ("window per tile", dict(kv_idx=widx, kv_cnt=wcnt, per_tile_walk=True)),
             ("routed", dict(kv_idx=ridx, kv_cnt=rcnt)),
             ("routed ordered", dict(kv_idx=ridx, kv_cnt=rcnt, work_order=order))]
    for name, kw in cases:
        o1, l1 = vsa.block_sparse_attn_fwd(lay, tq, tk, tv, want_lse=True, **kw)
        o2, l2 = vsa.block_sparse_attn_fwd(lay, tq, tk, vo, want_lse=True, v_operand=True, **kw)
        n1, m1 = vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, tv, want_lse=True, **kw)
        n2, m2 = vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, vo, want_lse=True, v_operand=True, **kw)
        torch.cuda.synchronize()
        assert _same(o1, o2) and torch.equal(l1, l2), name
        assert _same(n1, n2) and torch.equal(m1, m2), name


def test_full_size_layers_identical_with_v_operand():
    _gpu()
    for name in ("skiparse_768p", "window_480p", "topk32_16x32x32"):
        cfg = CONFIGS[name]
        _, blay = layouts(cfg)
        q, k, v = inputs(cfg.name)
        announce(f"bf16 V operand: full-size {name}")
        qn = to_device(q, "bf16")
        kt = vsa.tile_permute(blay, to_device(k, "bf16"))
        vn = to_device(v, "bf16")
        vt, vo = vsa.tile_permute(blay, vn), vsa.tile_permute_v(blay, vn)
        del vn
        walks = (False, True) if cfg.mask == "window" else (False,)
        if cfg.mask == "topk":
            _, qp = vsa.tile_permute_pool(blay, qn, means_only=True)
            _, kp = vsa.tile_permute_pool(blay, to_device(k, "bf16"), means_only=True)
            idx, cnt, _ = vsa.build_mask_topk_pooled(blay, qp, kp, top_k=cfg.top_k)
        else:
            idx, cnt = vsa.build_mask_window(blay, cfg.window if cfg.mask == "window" else (0, 0, 0))
        for per_tile in walks:
            o1, l1 = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, idx, cnt, want_lse=True,
                                                   per_tile_walk=per_tile)
            o2, l2 = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vo, idx, cnt, want_lse=True,
                                                   per_tile_walk=per_tile, v_operand=True)
            torch.cuda.synchronize()
            assert _same(o1, o2) and torch.equal(l1, l2), (name, per_tile)
            del o1, o2, l1, l2
        del qn, kt, vt, vo
        torch.cuda.empty_cache()
