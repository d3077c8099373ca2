"""Heavy-first work order for routed lists (FVAttn summary, Summary and
Abstract: Top-p routing makes the work per head and per query tile uneven).

* vsa_build_work_order against the order written out on the host: heads by
  total pairs, then query tiles by list length, both descending, ties in
  index order; counts clamped to [0, n_tiles];
* every routed forward (tiled bf16/fp8, natural bf16, natural fp8) gives the
  same bits with and without the order: it only changes which workgroup
  walks which query tile.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from synth import round_to_bf16
from tests.gpu_util import announce, lists_to_device, to_device

pytestmark = pytest.mark.gpu


def host_order(cnt: np.ndarray, n: int) -> np.ndarray:
    key = np.clip(cnt.reshape(-1, n).astype(np.int64), 0, n)
    tot = key.sum(axis=1)
    heads = np.lexsort((np.arange(len(tot)), -tot))
    return np.concatenate([bh * n + np.lexsort((np.arange(n), -key[bh])) for bh in heads]).astype(np.int32)


def test_order_matches_host_definition():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    announce("work order: random counts with ties, negatives and overlong counts")
    rng = np.random.default_rng(31)
    for (B, heads, T, H, W) in ((2, 3, 9, 14, 22), (1, 40, 21, 45, 80), (1, 1, 4, 4, 4), (3, 5, 1, 4, 260)):
        lay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=128, batch=B)
        n = vsa.layout_info(lay).n_tiles
        cnt = rng.integers(-3, n + 4, size=(B, heads, n)).astype(np.int32)
        cnt[0, 0, : n // 2] = 7                                     # a run of equal lengths
        if heads > 2:
            cnt[0, 2] = cnt[0, 1]                                   # two heads with equal totals
        order = vsa.build_work_order(lay, torch.from_numpy(cnt).cuda())
        torch.cuda.synchronize()
        got = order.cpu().numpy()
        assert np.array_equal(np.sort(got), np.arange(B * heads * n))
        assert np.array_equal(got, host_order(cnt, n))


def _routed_lists(rng, B, heads, n):
    idx = np.full((B, heads, n, n), -1, dtype=np.int32)
    cnt = np.zeros((B, heads, n), dtype=np.int32)
    for b in range(B):
        for h in range(heads):
            top = int(rng.integers(1, n + 1))                       # uneven heads
            for t in range(n):
                c = int(rng.integers(0, top + 1))
                idx[b, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                cnt[b, h, t] = c
    return idx, cnt


@pytest.mark.parametrize("tile,d", [((4, 4, 4), 128), ((4, 4, 4), 64), ((2, 4, 4), 128)])
def test_routed_forwards_identical_with_order(tile, d):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B, heads, T, H, W = 2, 3, 9, 14, 22
    lay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile, batch=B)
    info = vsa.layout_info(lay)
    n = info.n_tiles
    announce(f"work order: routed forwards tile={tile} d={d}")
    rng = np.random.default_rng(32)
    x = [round_to_bf16(rng.standard_normal((B, info.n_tokens, heads, d)).astype(np.float32))
         for _ in range(3)]
    nat = [to_device(a, "bf16") for a in x]
    tq, tk, tv = (vsa.tile_permute(lay, a) for a in nat)
    di, dc = lists_to_device(*_routed_lists(rng, B, heads, n))
    order = vsa.build_work_order(lay, dc)
    o1, l1 = vsa.block_sparse_attn_fwd(lay, tq, tk, tv, di, dc, want_lse=True)
    o2, l2 = vsa.block_sparse_attn_fwd(lay, tq, tk, tv, di, dc, want_lse=True, work_order=order)
    n1, m1 = vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, tv, di, dc, want_lse=True)
    n2, m2 = vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, tv, di, dc, want_lse=True, work_order=order)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(n1.view(torch.int16), n2.view(torch.int16)) and torch.equal(m1, m2)
    if tile == (4, 4, 4) and d == 128:
        (qc, qs), (kc, ks) = (vsa.quant_fp8_tiles(lay, a) for a in (tq, tk))
        vc, vs = vsa.quant_fp8_tiles(lay, tv, v_operand=True)
        f1, g1 = vsa.block_sparse_attn_fwd(lay, qc, kc, vc, di, dc, scales=(qs, ks, vs), want_lse=True,
                                           v_operand=True)
        f2, g2 = vsa.block_sparse_attn_fwd(lay, qc, kc, vc, di, dc, scales=(qs, ks, vs), want_lse=True,
                                           v_operand=True, work_order=order)
        h1, _ = vsa.block_sparse_attn_fwd_fp8_nat(lay, qc, kc, vc, (qs, ks, vs), di, dc, v_operand=True)
        h2, _ = vsa.block_sparse_attn_fwd_fp8_nat(lay, qc, kc, vc, (qs, ks, vs), di, dc, v_operand=True,
                                                  work_order=order)
        torch.cuda.synchronize()
        assert torch.equal(f1.view(torch.int16), f2.view(torch.int16)) and torch.equal(g1, g2)
        assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
