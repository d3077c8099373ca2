"""GPU parity: fp8 quantiser (bit-exact) and adaptive routing (exact up to near-ties)."""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import fp8 as OF
from oracle import layout as OL
from oracle import routing as OR
from oracle.layout import Layout as OLayout
from synth import CONFIGS, round_to_bf16
from tests.gpu_util import announce, inputs, layouts, to_device

pytestmark = pytest.mark.gpu

TIE = 1e-4        # near-tie band on oracle scores / cumulative mass


def _quant_check(x_nat, olay, blay):
    xd = to_device(x_nat, "bf16")
    xt = vsa.tile_permute(blay, xd)
    codes, scales = vsa.quant_fp8_tiles(blay, xt)
    torch.cuda.synchronize()
    rc, rs = OF.quantize_tiles(OL.permute(x_nat, olay), olay)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.int32), rs.view(np.int32))
    return codes, scales


def test_quant_small_edge_cases_bitexact():
    olay = OLayout(T=3, H=5, W=6, heads=2, head_dim=16, tile=(2, 4, 4))
    blay = vsa.Layout(T=3, H=5, W=6, heads=2, head_dim=16, tile=(2, 4, 4))
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, olay.n_tokens, 2, 16)).astype(np.float32) * 3
    x[0, :, 1, :] *= 1e-3                       # small values: subnormal codes
    x[0, :40, 0, :] = 0.0                       # makes tile 0 of head 0 all zero
    x[0, 41, 0, 3] = -0.0
    x = round_to_bf16(x)
    announce("quant small")
    _quant_check(x, olay, blay)


def test_quant_fp8_workload_bitexact():
    cfg = CONFIGS["fp8_topp_720p"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    for name, x in (("q", q), ("v", v)):
        announce(f"quant {cfg.name} {name}")
        codes, _ = _quant_check(x, olay, blay)
        codes2, _ = vsa.quant_fp8_tiles(blay, vsa.tile_permute(blay, to_device(x, "bf16")))
        torch.cuda.synchronize()
        assert torch.equal(codes, codes2)                   # deterministic


def test_quant_fp8_v_operand_bitexact():
    """vsa_quant_fp8_tiles_v: the oracle's codes in the P.V operand layout,
    the same scales; on a ragged grid with pads, an all-zero tile and
    subnormal codes, and on the 720p workload's V."""
    olay = OLayout(T=5, H=6, W=9, heads=2, head_dim=128, tile=(4, 4, 4))
    blay = vsa.Layout(T=5, H=6, W=9, heads=2, head_dim=128, tile=(4, 4, 4))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, olay.n_tokens, 2, 128)).astype(np.float32) * 2
    x[0, :, 1, :] *= 1e-3
    order = OL.token_order(olay).reshape(olay.n_tiles, 64)
    x[0, order[0][order[0] >= 0], 0, :] = 0.0         # tile 0 of head 0 all zero
    cases = [("ragged", round_to_bf16(x), olay, blay)]
    cfg = CONFIGS["fp8_topp_720p"]
    wo, wb = layouts(cfg)
    cases.append((cfg.name, inputs(cfg.name)[2], wo, wb))
    for name, xn, ol, bl in cases:
        announce(f"quant v-operand {name}")
        xt = vsa.tile_permute(bl, to_device(xn, "bf16"))
        codes, scales = vsa.quant_fp8_tiles(bl, xt, v_operand=True)
        torch.cuda.synchronize()
        rc, rs = OF.quantize_tiles(OL.permute(xn, ol), ol)
        assert np.array_equal(codes.cpu().numpy(), OF.v_operand_layout(rc, ol))
        assert np.array_equal(scales.cpu().numpy().view(np.int32), rs.view(np.int32))


def test_quant_fp8_v_operand_rejects_other_shapes():
    lay = vsa.Layout(T=3, H=5, W=6, heads=2, head_dim=16, tile=(2, 4, 4))
    x = torch.zeros((1, 2, vsa.layout_info(lay).n_padded, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vsa.VsaError):
        vsa.quant_fp8_tiles(lay, x, v_operand=True)


def _accept_topk(gpu_row, ref_row, s, k):
    if gpu_row == ref_row:
        return True
    order = sorted(range(len(s)), key=lambda j: (-s[j], j))
    kth = s[order[min(k, len(order)) - 1]]
    diff = set(gpu_row) ^ set(ref_row)
    return len(gpu_row) == len(ref_row) and all(abs(s[j] - kth) <= TIE for j in diff)


def _accept_topp(gpu_row, s, p, floor):
    """GPU row acceptable under the top-p rule given oracle scores s (fp64).

    Returns False, "count" (the row keeps the oracle's count and differs only
    by swaps between tiles whose oracle scores lie within TIE of the cut) or
    "mass" (the count differs by one, admitted because the oracle's cumulative
    mass at the cut lies within TIE of p: the mass-tie reading)."""
    order = sorted([j for j in range(len(s)) if np.isfinite(s[j])], key=lambda j: (-s[j], j))
    vals = np.array([s[j] for j in order])
    w = np.exp(vals - vals.max())
    cum = np.cumsum(w / w.sum())
    n = len(order)
    hit = np.nonzero(cum >= p)[0]
    c = int(hit[0]) + 1 if hit.size else n
    c = min(max(c, floor), n)
    allowed = {c}
    if c - 1 >= max(floor, 1) and cum[c - 2] >= p - TIE:
        allowed.add(c - 1)
    if c + 1 <= n and cum[c - 1] <= p + TIE:
        allowed.add(c + 1)
    m = len(gpu_row)
    if m not in allowed or gpu_row != sorted(gpu_row):
        return False
    ref = set(order[:m])
    cut = s[order[m - 1]]
    if not all(abs(s[j] - cut) <= TIE for j in set(gpu_row) ^ ref):
        return False
    return "count" if m == c else "mass"


def _oracle_scores(cfg, olay, q, k):
    qb = OR.pool_tiles(OL.permute(q, olay), olay)
    kb = OR.pool_tiles(OL.permute(k, olay), olay)
    return OR.coarse_scores(qb, kb, 1.0 / math.sqrt(cfg.head_dim))


def test_topk_routing_workload():
    cfg = CONFIGS["topk32_16x32x32"]
    olay, blay = layouts(cfg)
    q, k, _ = inputs(cfg.name)
    announce(f"route topk {cfg.name}")
    qd = vsa.tile_permute(blay, to_device(q, "bf16"))
    kd = vsa.tile_permute(blay, to_device(k, "bf16"))
    kv_idx, kv_cnt, scores = vsa.build_mask_topk(blay, qd, kd, top_k=cfg.top_k, want_scores=True)
    torch.cuda.synchronize()
    s = _oracle_scores(cfg, olay, q, k)
    assert np.allclose(scores.cpu().numpy(), s, rtol=0, atol=1e-4)
    ridx, rcnt = OR.select_lists_vectorized(s, top_k=cfg.top_k)
    gi, gc = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    assert np.array_equal(gc, rcnt)
    bad = 0
    for h in range(cfg.heads):
        for i in range(olay.n_tiles):
            g = gi[0, h, i, :gc[0, h, i]].tolist()
            r = ridx[0, h, i, :rcnt[0, h, i]].tolist()
            bad += not _accept_topk(g, r, s[0, h, i], cfg.top_k)
    assert bad == 0
    kv_idx2, kv_cnt2, _ = vsa.build_mask_topk(blay, qd, kd, top_k=cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(kv_idx, kv_idx2) and torch.equal(kv_cnt, kv_cnt2)


def test_topp_routing_workload():
    cfg = CONFIGS["fp8_topp_720p"]
    olay, blay = layouts(cfg)
    q, k, _ = inputs(cfg.name)
    announce(f"route topp {cfg.name}")
    qd = vsa.tile_permute(blay, to_device(q, "bf16"))
    kd = vsa.tile_permute(blay, to_device(k, "bf16"))
    kv_idx, kv_cnt, _ = vsa.build_mask_topk(blay, qd, kd, top_p=cfg.top_p, k_floor=cfg.k_floor)
    torch.cuda.synchronize()
    s = _oracle_scores(cfg, olay, q, k)
    gi, gc = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    ridx, rcnt = OR.select_lists_vectorized(s, top_p=cfg.top_p, k_floor=cfg.k_floor)
    bad = []
    admitted = {"count": 0, "mass": 0}
    for h in range(cfg.heads):
        for i in range(olay.n_tiles):
            g = gi[0, h, i, :gc[0, h, i]].tolist()
            if gc[0, h, i] == rcnt[0, h, i] and g == ridx[0, h, i, :rcnt[0, h, i]].tolist():
                continue
            why = _accept_topp(g, s[0, h, i], cfg.top_p, cfg.k_floor)
            if not why:
                bad.append((h, i))
            else:
                admitted[why] += 1
    assert not bad, f"{len(bad)} rows differ beyond near-ties, e.g. {bad[:5]}"
    # the mass-tie reading may not widen silently: at this workload it admits
    # a few tens of the 57,600 rows (measured: 16, and 2 by score near-ties); at most 0.1% pass
    print(f"[route topp] rows admitted by score near-ties: {admitted['count']}, "
          f"by mass near-ties (count +-1): {admitted['mass']}", file=sys.stderr)
    assert admitted["mass"] <= gc.size // 1000
    assert admitted["count"] <= gc.size // 1000
    assert int(gc.min()) >= cfg.k_floor


# ---- tile permute with the pool folded in (FVAttn summary: video-aware block
# organisation; VSA page, Research Type row: the coarse stage on pooled blocks)

def _pool_bound(x_tiled, olay):
    """Worst-case fp32 error of a tile mean of n <= 64 values summed in any
    order: (n - 1) u sum|x| / n < 64 u mean|x|, plus the final division's u |mean|."""
    return 64 * 2.0 ** -24 * OR.pool_tiles(np.abs(x_tiled), olay)


def _check_permute_pool(olay, blay, x, route):
    """x natural-order float32 (bf16 values). Tiled copy bit-identical to the
    plain permute, means against the oracle, routing from the means
    bit-identical to routing from the tiled tensors."""
    xd = [to_device(a, "bf16") for a in x]
    outs = [vsa.tile_permute_pool(blay, a) for a in xd]
    plain = [vsa.tile_permute(blay, a) for a in xd]
    torch.cuda.synchronize()
    for (t, p), ref_t, a in zip(outs, plain, x):
        assert torch.equal(t.view(torch.int16), ref_t.view(torch.int16))
        xt = OL.permute(a, olay)
        ref = OR.pool_tiles(xt, olay)
        got = p.cpu().numpy()
        fin = np.isfinite(ref)
        assert np.all(got[~fin] == 0.0)
        bound = _pool_bound(xt, olay) + 2.0 ** -24 * np.abs(np.nan_to_num(ref))
        assert np.all(np.abs(got[fin] - ref[fin]) <= bound[fin] + 1e-30)
    (qt, qp), (kt, kp) = outs
    a = vsa.build_mask_topk(blay, qt, kt, want_scores=True, **route)
    b = vsa.build_mask_topk_pooled(blay, qp, kp, want_scores=True, **route)
    torch.cuda.synchronize()
    # slots past a row's count are not written: compare the counts and the lists
    assert torch.equal(a[1], b[1])
    valid = torch.arange(a[0].shape[-1], device=a[0].device) < a[1].unsqueeze(-1)
    assert torch.equal(a[0][valid], b[0][valid])
    assert torch.equal(a[2].view(torch.int32), b[2].view(torch.int32))
    return b


@pytest.mark.parametrize("shape,tile,kind,stride,batch,d", [
    ((5, 9, 13), (2, 4, 4), "tile3d", (2, 2), 2, 64),
    ((3, 4, 6), (1, 4, 4), "skiparse2d", (2, 2), 1, 128),
    ((2, 6, 9), (1, 4, 8), "skiparse2d", (3, 3), 2, 96),
])
def test_permute_pool_ragged(shape, tile, kind, stride, batch, d):
    T, H, W = shape
    heads = 3
    olay = OLayout(T=T, H=H, W=W, heads=heads, head_dim=d, kind=kind, tile=tile, stride=stride)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind=kind, tile=tile, stride=stride,
                      batch=batch)
    rng = np.random.default_rng(3301 + d)
    x = [round_to_bf16((rng.standard_normal((batch, T * H * W, heads, d)) * 2.0 + 0.5)
                       .astype(np.float32)) for _ in range(2)]
    announce(f"permute+pool {shape} tile={tile} {kind} B={batch} d={d}")
    top_k = min(3, olay.n_tiles)
    kv_idx, kv_cnt, scores = _check_permute_pool(olay, blay, x, dict(top_k=top_k))
    s = OR.coarse_scores(OR.pool_tiles(OL.permute(x[0], olay), olay),
                         OR.pool_tiles(OL.permute(x[1], olay), olay), 1.0 / math.sqrt(d))
    ridx, rcnt = OR.select_lists_vectorized(s, top_k=top_k)
    gi, gc = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    assert np.array_equal(gc, rcnt)
    for b in range(batch):
        for h in range(heads):
            for i in range(olay.n_tiles):
                g = gi[b, h, i, :gc[b, h, i]].tolist()
                r = ridx[b, h, i, :rcnt[b, h, i]].tolist()
                assert _accept_topk(g, r, s[b, h, i], top_k), (b, h, i)


@pytest.mark.parametrize("name", ["topk32_16x32x32", "fp8_topp_720p"])
def test_permute_pool_workloads(name):
    cfg = CONFIGS[name]
    olay, blay = layouts(cfg)
    q, k, _ = inputs(cfg.name)
    announce(f"permute+pool {cfg.name}")
    route = dict(top_k=cfg.top_k) if cfg.top_p <= 0 else dict(top_p=cfg.top_p, k_floor=cfg.k_floor)
    _check_permute_pool(olay, blay, (q, k), route)
