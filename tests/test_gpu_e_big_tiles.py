"""GPU parity for big tiles (FPSAttention, Approach and ablation table:
(6,8,8) tiles built from (1,8,8) ones, windows such as (6,6,1), FP8 scales
on the same big tiles): grouped window lists and grouped e4m3 codes and
scales are integer / exactly rounded work, so bit-exact against the oracle;
attention over the grouped lists keeps the forward's gates (bf16 max-abs
2e-2 and relative L2 1e-2; fp8 relative L2 5e-2 against the oracle of the
fp8 method)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import layout as OL
from oracle import masks as OM
from synth import CONFIGS, round_to_bf16
from tests.gpu_util import announce, errors, inputs, to_device

pytestmark = pytest.mark.gpu

BIG = (6, 1, 1)            # (6,8,8) big tiles from (1,8,8) tiles


def _layouts(T, H, W, heads, tile=(1, 8, 8), d=128):
    return (OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile),
            vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile))


@pytest.mark.parametrize("shape,tile,group,ext", [
    ((21, 30, 52), (1, 8, 8), BIG, (6, 6, 6)),
    ((21, 30, 52), (1, 8, 8), BIG, (6, 6, 1)),
    ((21, 30, 52), (1, 8, 8), BIG, (3, 3, 1)),
    ((21, 45, 80), (1, 8, 8), BIG, (2, 3, 4)),
    ((5, 9, 13), (2, 4, 4), (2, 2, 3), (1, 2, 3)),
])
def test_grouped_window_lists_bitexact(shape, tile, group, ext):
    olay, blay = _layouts(*shape, heads=1, tile=tile)
    announce(f"grouped window {shape} tile={tile} group={group} ext={ext}")
    idx, cnt = vsa.build_mask_window_grouped(blay, group, ext)
    torch.cuda.synchronize()
    ref = OM.window_lists_grouped(olay, group, ext)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for t, row in enumerate(ref):
        assert cnt[t] == len(row) and idx[t, :cnt[t]].tolist() == row, t


@pytest.mark.parametrize("group,vop", [(BIG, False), (BIG, True), ((2, 2, 3), False)])
def test_grouped_quantiser_bitexact(group, vop):
    olay, blay = _layouts(21, 30, 52, heads=3)
    rng = np.random.default_rng(2601 + 7 * vop + group[1])
    x = round_to_bf16((rng.standard_normal((1, olay.n_tokens, 3, 128)) *
                       rng.uniform(0.2, 3.0, size=(1, 1, 3, 1))).astype(np.float32))
    announce(f"grouped quantiser group={group} v_operand={vop}")
    xt = vsa.tile_permute(blay, to_device(x, "bf16"))
    codes, scales = vsa.quant_fp8_tiles_grouped(blay, xt, group, v_operand=vop)
    torch.cuda.synchronize()
    rc, rs = OF.quantize_tiles_grouped(OL.permute(x, olay), olay, group)
    if vop:
        rc = OF.v_operand_layout(rc, olay)
    assert np.array_equal(scales.cpu().numpy().view(np.int32), rs.view(np.int32))
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.fixture(scope="module")
def big_case():
    """The 480p window workload's inputs on (1,8,8) tiles, 12 heads."""
    cfg = CONFIGS["window_480p"]
    q, k, v = inputs(cfg.name)
    olay, blay = _layouts(cfg.T, cfg.H, cfg.W, heads=cfg.heads)
    dev = [vsa.tile_permute(blay, to_device(x, "bf16")) for x in (q, k, v)]
    host = [OL.permute(x, olay).astype(np.float64) for x in (q, k, v)]
    return olay, blay, dev, host


def _items(olay, n, seed):
    rng = np.random.default_rng(seed)
    return sorted({(0, int(h), int(t)) for h, t in zip(rng.integers(0, olay.heads, n),
                                                       rng.integers(0, olay.n_tiles, n))}
                  | {(0, 0, 0), (0, olay.heads - 1, olay.n_tiles - 1)})


def _gather(x, olay, items):
    C = olay.tile_tokens
    return np.concatenate([x[b, h, t * C:(t + 1) * C] for b, h, t in items])


@pytest.mark.parametrize("ext,per_tile", [((6, 6, 6), False), ((6, 6, 1), False), ((6, 6, 1), True)])
def test_attention_over_grouped_windows_bf16(big_case, ext, per_tile):
    olay, blay, (qd, kd, vd), host = big_case
    announce(f"attention bf16 over grouped windows {ext} per_tile_walk={per_tile}")
    idx, cnt = vsa.build_mask_window_grouped(blay, BIG, ext)
    out, _ = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, idx, cnt, per_tile_walk=per_tile)
    torch.cuda.synchronize()
    lists = OM.window_lists_grouped(olay, BIG, ext)
    items = _items(olay, 40, 2700 + ext[2])
    O, _ = OA.attention(*host, olay, OA.shared_lists(lists), 1.0 / math.sqrt(128), items=items)
    mae, rl2 = errors(_gather(out.float().cpu().numpy(), olay, items), _gather(O, olay, items))
    print(f"max_abs={mae:.3e} rel_l2={rl2:.3e}")
    assert mae <= 2e-2 and rl2 <= 1e-2


@pytest.mark.parametrize("per_tile", [False, True])
def test_attention_over_grouped_windows_fp8_grouped_scales(big_case, per_tile):
    """fp8 attention with one scale per (6,8,8) tile (V in the P.V operand
    layout), against the oracle of the fp8 method: the oracle's grouped
    quantiser, dequantisation, fp64 attention over the same lists."""
    olay, blay, (qd, kd, vd), host = big_case
    ext = (6, 6, 1)
    announce("attention fp8 over grouped windows, grouped scales")
    idx, cnt = vsa.build_mask_window_grouped(blay, BIG, ext)
    (qc, qs), (kc, ks) = (vsa.quant_fp8_tiles_grouped(blay, x, BIG) for x in (qd, kd))
    vc, vs = vsa.quant_fp8_tiles_grouped(blay, vd, BIG, v_operand=True)
    out, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, idx, cnt, scales=(qs, ks, vs), v_operand=True,
                                       per_tile_walk=per_tile)
    torch.cuda.synchronize()
    deq = [OF.dequantize_tiles(*OF.quantize_tiles_grouped(x.astype(np.float32), olay, BIG), olay)
           for x in host]
    lists = OM.window_lists_grouped(olay, BIG, ext)
    items = _items(olay, 30, 2801)
    O, _ = OA.attention(*deq, olay, OA.shared_lists(lists), 1.0 / math.sqrt(128), items=items)
    mae, rl2 = errors(_gather(out.float().cpu().numpy(), olay, items), _gather(O, olay, items))
    print(f"max_abs={mae:.3e} rel_l2={rl2:.3e}")
    assert rl2 <= 5e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_per_tile_walk_matches_grouped_walk(dtype):
    """list_mode 2 walks the same shared table per query tile: the output
    equals the grouped walk's to rounding order, and the lse likewise."""
    T, H, W, heads, d = 7, 10, 13, 2, 128
    olay, blay = _layouts(T, H, W, heads, tile=(4, 4, 4), d=d)
    rng = np.random.default_rng(2901 + (dtype == "f32"))
    xs = [rng.standard_normal((1, olay.n_tokens, heads, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        xs = [round_to_bf16(x) for x in xs]
    qd, kd, vd = (vsa.tile_permute(blay, to_device(x, dtype)) for x in xs)
    idx, cnt = vsa.build_mask_window(blay, (1, 1, 1))
    announce(f"per-tile walk vs grouped walk {dtype}")
    o1, l1 = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, idx, cnt, want_lse=True)
    o2, l2 = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, idx, cnt, want_lse=True, per_tile_walk=True)
    torch.cuda.synchronize()
    mae, rl2 = errors(o2.float().cpu().numpy(), o1.float().cpu().numpy().astype(np.float64))
    assert mae <= 1e-2 and rl2 <= 5e-3
    a, b = l1.cpu().numpy(), l2.cpu().numpy()
    fin = np.isfinite(a)
    assert np.array_equal(fin, np.isfinite(b)) and np.abs(a[fin] - b[fin]).max() <= 2e-3
