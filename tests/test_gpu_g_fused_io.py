"""The fused natural-order calls against the unfused path they replace
(FVAttn summary: video-aware block organisation; FPSAttention, Approach:
FP8 on the shared tiles): bit-identical results.

* vsa_quant_fp8_tiles_nat = vsa_tile_permute then vsa_quant_fp8_tiles(_v),
  its tile means = vsa_tile_permute_pool's;
* vsa_tile_permute_pool with no tiled copy = the same means;
* vsa_block_sparse_attn_fwd_fp8_nat = vsa_block_sparse_attn_fwd then
  vsa_tile_permute(inverse), with the same lse.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import layout as OL
from oracle import masks as OM
from synth import CONFIGS, round_to_bf16
from tests.gpu_util import announce, inputs, layouts, lists_to_device, table_from_lists, to_device

pytestmark = pytest.mark.gpu

SMALL = [  # (T, H, W, kind, tile, stride, d, batch)
    ((5, 9, 13), "tile3d", (4, 4, 4), (1, 1), 128, 2),
    ((3, 6, 10), "skiparse2d", (4, 4, 4), (2, 2), 128, 1),
    ((4, 8, 8), "tile3d", (2, 4, 4), (1, 1), 64, 1),
    ((6, 8, 9), "tile3d", (4, 4, 4), (1, 1), 96, 1),
    ((5, 8, 8), "tile3d", (4, 4, 4), (1, 1), 256, 1),
]


def _check_quant_nat(blay, xd):
    t = vsa.tile_permute(blay, xd)
    _, pooled_ref = vsa.tile_permute_pool(blay, xd)
    _, pooled_only = vsa.tile_permute_pool(blay, xd, means_only=True)
    c_ref, s_ref = vsa.quant_fp8_tiles(blay, t)
    c, s, p = vsa.quant_fp8_tiles_nat(blay, xd, want_pooled=True)
    c2, s2, p2 = vsa.quant_fp8_tiles_nat(blay, xd)
    torch.cuda.synchronize()
    assert torch.equal(c, c_ref) and torch.equal(c2, c_ref)
    assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32)) and torch.equal(s2, s_ref)
    assert torch.equal(p.view(torch.int32), pooled_ref.view(torch.int32))
    assert torch.equal(pooled_only.view(torch.int32), pooled_ref.view(torch.int32))
    assert p2 is None
    if blay.tile == (4, 4, 4) and blay.head_dim == 128:
        v_ref, vs_ref = vsa.quant_fp8_tiles(blay, t, v_operand=True)
        v, vs, _ = vsa.quant_fp8_tiles_nat(blay, xd, v_operand=True)
        torch.cuda.synchronize()
        assert torch.equal(v, v_ref) and torch.equal(vs, vs_ref)


@pytest.mark.parametrize("grid,kind,tile,stride,d,batch", SMALL)
def test_quant_nat_small_grids(grid, kind, tile, stride, d, batch):
    T, H, W = grid
    blay = vsa.Layout(T=T, H=H, W=W, heads=3, head_dim=d, kind=kind, tile=tile, stride=stride,
                      batch=batch)
    rng = np.random.default_rng(77)
    x = round_to_bf16(rng.standard_normal((batch, T * H * W, 3, d)).astype(np.float32) * 3)
    x[0, :5] = 0.0                                          # an all-zero stretch of tokens
    announce(f"quant nat {grid} {kind} {tile} d={d} B={batch}")
    _check_quant_nat(blay, to_device(x, "bf16"))


def test_quant_nat_topp_720p():
    cfg = CONFIGS["fp8_topp_720p"]
    _, blay = layouts(cfg)
    q, _, _ = inputs(cfg.name)
    announce("quant nat 720p, 40 heads")
    _check_quant_nat(blay, to_device(q, "bf16"))


def _fp8_nat_case(blay, olay, lists_idx, lists_cnt, seed):
    rng = np.random.default_rng(seed)
    x = [round_to_bf16(rng.standard_normal((blay.batch, olay.n_tokens, blay.heads, 128)).astype(np.float32))
         for _ in range(3)]
    xd = [to_device(a, "bf16") for a in x]
    (qc, qs, _), (kc, ks, _) = (vsa.quant_fp8_tiles_nat(blay, a) for a in xd[:2])
    vc, vs, _ = vsa.quant_fp8_tiles_nat(blay, xd[2], v_operand=True)
    di, dc = lists_idx, lists_cnt
    for vop in (False, True):
        vv, vvs = (vc, vs) if vop else vsa.quant_fp8_tiles(blay, vsa.tile_permute(blay, xd[2]))
        ref, lref = vsa.block_sparse_attn_fwd(blay, qc, kc, vv, di, dc, scales=(qs, ks, vvs),
                                              v_operand=vop, want_lse=True)
        ref_nat = vsa.tile_permute(blay, ref, inverse=True)
        out = torch.full_like(ref_nat, 5.0)
        out, lse = vsa.block_sparse_attn_fwd_fp8_nat(blay, qc, kc, vv, (qs, ks, vvs), di, dc,
                                                     v_operand=vop, want_lse=True, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_nat.view(torch.int16)), vop
        assert torch.equal(lse, lref)


@pytest.mark.parametrize("mode", ["routed", "shared"])
def test_fp8_natural_out_ragged(mode):
    T, H, W, heads = 9, 14, 22, 2
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=128, tile=(4, 4, 4), batch=2)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=128, tile=(4, 4, 4), batch=2)
    n = olay.n_tiles
    announce(f"fp8 natural out {mode}")
    if mode == "shared":
        di, dc = lists_to_device(*table_from_lists(OM.window_lists(olay, 1, 1, 1)))
    else:
        rng = np.random.default_rng(5)
        idx = np.full((2, heads, n, n), -1, dtype=np.int32)
        cnt = np.zeros((2, heads, n), dtype=np.int32)
        for b in range(2):
            for h in range(heads):
                for t in range(n):
                    c = int(rng.integers(0, n // 2))
                    idx[b, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                    cnt[b, h, t] = c
        di, dc = lists_to_device(idx, cnt)
    _fp8_nat_case(blay, olay, di, dc, 99)


def test_fp8_natural_out_topp_720p():
    """The 720p top-p layer as the bench runs it, fused: quantisers from the
    natural order, routing from their means, fp8 walk with natural O."""
    cfg = CONFIGS["fp8_topp_720p"]
    _, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    announce("fp8 natural out 720p top-p, fused pipeline vs unfused")
    qn, kn, vn = (to_device(x, "bf16") for x in (q, k, v))
    # unfused: permute + pool, route, quantise the tiled copies, attention, unpermute
    (tq, qp), (tk, kp) = (vsa.tile_permute_pool(blay, x) for x in (qn, kn))
    tv = vsa.tile_permute(blay, vn)
    idx, cnt, _ = vsa.build_mask_topk_pooled(blay, qp, kp, top_p=cfg.top_p, k_floor=cfg.k_floor)
    (qc, qs), (kc, ks), (vc, vs) = (vsa.quant_fp8_tiles(blay, x, v_operand=vop)
                                    for x, vop in ((tq, False), (tk, False), (tv, True)))
    ref, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, idx, cnt, scales=(qs, ks, vs), v_operand=True)
    ref = vsa.tile_permute(blay, ref, inverse=True)
    del tq, tk, tv, qc, kc, vc
    # fused
    (qc2, qs2, qp2), (kc2, ks2, kp2) = (vsa.quant_fp8_tiles_nat(blay, x, want_pooled=True) for x in (qn, kn))
    vc2, vs2, _ = vsa.quant_fp8_tiles_nat(blay, vn, v_operand=True)
    idx2, cnt2, _ = vsa.build_mask_topk_pooled(blay, qp2, kp2, top_p=cfg.top_p, k_floor=cfg.k_floor)
    out, _ = vsa.block_sparse_attn_fwd_fp8_nat(blay, qc2, kc2, vc2, (qs2, ks2, vs2), idx2, cnt2, v_operand=True)
    torch.cuda.synchronize()
    assert torch.equal(cnt2, cnt)
    slot = torch.arange(idx.shape[-1], device=idx.device)
    used = slot[None, None, None, :] < cnt[..., None]          # slots past a count are unspecified
    assert torch.equal(torch.where(used, idx2, 0), torch.where(used, idx, 0))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # the heavy-first dealing the bench uses changes nothing in the output
    from tests.test_gpu_h_work_order import host_order
    order = vsa.build_work_order(blay, cnt2)
    out2, _ = vsa.block_sparse_attn_fwd_fp8_nat(blay, qc2, kc2, vc2, (qs2, ks2, vs2), idx2, cnt2, v_operand=True,
                                                work_order=order)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), host_order(cnt2.cpu().numpy(), cnt2.shape[-1]))
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))
