"""GPU parity at the full workload sizes, through the launches bench.py times:
every query tile of one head (several hundred thousand output rows each)
against the fp64 oracle.

* 768p Skiparse sparse layer (OSP-Next card, Model Summary: Skiparse-2D along
  H and W): natural-order Q in, natural-order O out (vsa_block_sparse_attn_fwd_nat),
  V in the bf16 P.V operand layout (vsa_tile_permute_v) as the bench runs it,
  Skiparse lists from vsa_build_mask_window, 40 heads; the oracle checks every
  one of the 1,260 query tiles of one head.
* 768p dense layer (OSP-Next wiki TL;DR: hybrid full + sparse): 256 query
  tiles of one head against all 80,640 keys.
* 720p top-p fp8 layer, the bench's exact pipeline (FVAttn summary: Top-p
  routing with a Top-k floor; FPSAttention, Approach: FP8 on the shared
  tiles): permute + pool of Q and K, permute of V, routing from the means,
  e4m3 quantisation (V in the P.V operand layout), fp8 attention over the
  routed lists. The head with the fewest listed tiles: its lists against the
  oracle's routing (exact up to near-ties), its output and lse for every query
  tile against the oracle of the fp8 method on those lists.
* 480p window layer walked per query tile (list_mode 2), every tile of one head.
* top-32 layer through the bench's calls (VSA page, Research Type row: a
  coarse stage picks key blocks per query block): means of Q without a
  tiled copy, permute + pool of K, V into the bf16 operand layout, routing
  from the means, one-tile walks with natural-order Q and O; one head's lists
  against the oracle's routing (near-ties excepted) and every query tile of
  it against the oracle on the GPU's lists.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import layout as OL
from oracle import masks as OM
from oracle import routing as OR
from synth import CONFIGS
from tests.gpu_util import announce, errors, inputs, layouts, to_device
from tests.test_gpu_b_quant_route import _accept_topk, _accept_topp

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2, REL_L2_FP8, LSE_BF16 = 2e-2, 1e-2, 5e-2, 2e-3


def _one_head(cfg, x, h):
    """Natural-order float32 [1, N, heads, d] -> the oracle's tiled fp64 copy of head h."""
    olay1 = OL.Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=1, head_dim=cfg.head_dim, kind=cfg.kind,
                      tile=cfg.tile, stride=cfg.stride)
    return olay1, OL.permute(np.ascontiguousarray(x[:, :, [h]]), olay1).astype(np.float64)


def _gate(g, r, lse_g, lse_r, what, rel=REL_L2, mae_gate=MAX_ABS, lse_gate=LSE_BF16):
    mae, rl2 = errors(g, r)
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isfinite(lse_g), fin), what
    lerr = float(np.abs(lse_g[fin] - lse_r[fin]).max())
    print(f"{what}: max_abs={mae:.3e} rel_l2={rl2:.3e} lse_max_abs={lerr:.3e}")
    assert mae <= mae_gate and rl2 <= rel, (what, mae, rl2)
    assert lerr <= lse_gate, (what, lerr)


def _skiparse_case():
    cfg = CONFIGS["skiparse_768p"]
    _, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    qn = to_device(q, "bf16")
    kt = vsa.tile_permute(blay, to_device(k, "bf16"))
    vt = vsa.tile_permute_v(blay, to_device(v, "bf16"))       # V in the P.V operand layout
    return cfg, blay, (q, k, v), qn, kt, vt


def test_skiparse_768p_sparse_every_tile_of_one_head():
    cfg, blay, (q, k, v), qn, kt, vt = _skiparse_case()
    h = 17
    announce("full-size: 768p Skiparse sparse layer, natural-order I/O, head 17, all 1,260 tiles")
    idx, cnt = vsa.build_mask_window(blay, (0, 0, 0))
    out, lse = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, idx, cnt, want_lse=True, v_operand=True)
    torch.cuda.synchronize()
    olay1, qo = _one_head(cfg, q, h)
    _, ko = _one_head(cfg, k, h)
    _, vo = _one_head(cfg, v, h)
    O, L = OA.attention(qo, ko, vo, olay1, OA.shared_lists(OM.skiparse_lists(olay1)),
                        1.0 / math.sqrt(cfg.head_dim))
    g = OL.permute(out[:, :, [h]].float().cpu().numpy(), olay1)        # natural -> tiled, head h
    real = OL.token_order(olay1) >= 0
    _gate(g[0, 0, real], O[0, 0, real], lse[0, h].cpu().numpy(), L[0, 0], "skiparse sparse head 17")


def test_skiparse_768p_dense_256_tiles_of_one_head():
    cfg, blay, (q, k, v), qn, kt, vt = _skiparse_case()
    h = 29
    announce("full-size: 768p dense layer, natural-order I/O, head 29, 256 query tiles")
    out, lse = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, want_lse=True, v_operand=True)
    torch.cuda.synchronize()
    olay1, qo = _one_head(cfg, q, h)
    _, ko = _one_head(cfg, k, h)
    _, vo = _one_head(cfg, v, h)
    rng = np.random.default_rng(29)
    tiles = sorted(rng.choice(olay1.n_tiles, 256, replace=False).tolist())
    items = [(0, 0, t) for t in tiles]
    O, L = OA.attention(qo, ko, vo, olay1, OA.shared_lists(OM.dense_lists(olay1)),
                        1.0 / math.sqrt(cfg.head_dim), items=items)
    g = OL.permute(out[:, :, [h]].float().cpu().numpy(), olay1)
    C = olay1.tile_tokens
    rows = np.concatenate([np.arange(t * C, (t + 1) * C) for t in tiles])
    lg = lse[0, h].cpu().numpy()
    _gate(g[0, 0, rows], O[0, 0, rows], lg[rows], L[0, 0, rows], "skiparse dense head 29, 256 tiles")


def test_topp_720p_fp8_bench_pipeline_every_tile_of_one_head():
    cfg = CONFIGS["fp8_topp_720p"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    announce("full-size: 720p top-p fp8 pipeline (permute+pool, routing, quantisers, fp8 walk)")
    (tq, qp), (tk, kp) = (vsa.tile_permute_pool(blay, to_device(x, "bf16")) for x in (q, k))
    tv = vsa.tile_permute(blay, to_device(v, "bf16"))
    idx, cnt, _ = vsa.build_mask_topk_pooled(blay, qp, kp, top_p=cfg.top_p, k_floor=cfg.k_floor)
    (qc, qs), (kc, ks), (vc, vs) = (vsa.quant_fp8_tiles(blay, x, v_operand=vop)
                                    for x, vop in ((tq, False), (tk, False), (tv, True)))
    out, lse = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, idx, cnt, scales=(qs, ks, vs),
                                         v_operand=True, want_lse=True)
    torch.cuda.synchronize()
    gc = cnt.cpu().numpy()
    h = int(np.argmin(gc[0].sum(axis=1)))          # the head with the fewest listed tiles
    gi = idx[0, h].cpu().numpy()
    olay1, qo = _one_head(cfg, q, h)
    _, ko = _one_head(cfg, k, h)
    _, vo = _one_head(cfg, v, h)
    # the head's routed lists against the oracle's routing (near-ties excepted)
    s = OR.coarse_scores(OR.pool_tiles(qo, olay1), OR.pool_tiles(ko, olay1), 1.0 / math.sqrt(cfg.head_dim))
    ridx, rcnt = OR.select_lists_vectorized(s, top_p=cfg.top_p, k_floor=cfg.k_floor)
    lists = [gi[t, :gc[0, h, t]].tolist() for t in range(olay1.n_tiles)]
    bad = [t for t in range(olay1.n_tiles)
           if not (lists[t] == ridx[0, 0, t, :rcnt[0, 0, t]].tolist()
                   or _accept_topp(lists[t], s[0, 0, t], cfg.top_p, cfg.k_floor))]
    assert not bad, f"head {h}: {len(bad)} lists differ beyond near-ties"
    # every query tile of that head against the oracle of the fp8 method on the GPU's lists
    deq = [OF.dequantize_tiles(*OF.quantize_tiles(x.astype(np.float32), olay1), olay1) for x in (qo, ko, vo)]
    sigma = 1.0 / math.sqrt(cfg.head_dim)
    Od, Ld = OA.attention(*deq, olay1, OA.shared_lists(lists), sigma)
    Ou, _ = OA.attention(qo, ko, vo, olay1, OA.shared_lists(lists), sigma)
    real = OL.token_order(olay1) >= 0
    g = out[0, h].float().cpu().numpy()[real]
    mae_d, rl2_d = errors(g, Od[0, 0, real])
    _, rl2_u = errors(g, Ou[0, 0, real])
    _, rl2_q = errors(Od[0, 0, real], Ou[0, 0, real])
    lg = lse[0, h].cpu().numpy()
    fin = np.isfinite(Ld[0, 0])
    assert np.array_equal(np.isfinite(lg), fin)
    lerr = float(np.abs(lg[fin] - Ld[0, 0][fin]).max())
    print(f"top-p fp8 head {h} ({int(gc[0, h].sum())} listed tiles): vs fp8-method oracle "
          f"max_abs={mae_d:.3e} rel_l2={rl2_d:.3e} lse_max_abs={lerr:.3e}; vs bf16 oracle "
          f"rel_l2={rl2_u:.3e}; quantisation alone rel_l2={rl2_q:.3e}")
    assert rl2_d <= REL_L2_FP8
    assert rl2_u <= 1.1 * rl2_q + 5e-3
    # one-tile walk: the row sums are the exact fp32 sums of the unrounded weights, so
    # lse follows the dequantised oracle to fp32 rounding of the scores and the exp2
    assert lerr <= 2e-3


def test_window_480p_per_tile_walk_every_tile_of_one_head():
    cfg = CONFIGS["window_480p"]
    _, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    h = 5
    announce("full-size: 480p window layer walked per query tile, head 5, all 624 tiles")
    qn = to_device(q, "bf16")
    kt = vsa.tile_permute(blay, to_device(k, "bf16"))
    vt = vsa.tile_permute_v(blay, to_device(v, "bf16"))
    idx, cnt = vsa.build_mask_window(blay, cfg.window)
    out, lse = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, idx, cnt, want_lse=True, per_tile_walk=True,
                                             v_operand=True)
    torch.cuda.synchronize()
    olay1, qo = _one_head(cfg, q, h)
    _, ko = _one_head(cfg, k, h)
    _, vo = _one_head(cfg, v, h)
    O, L = OA.attention(qo, ko, vo, olay1, OA.shared_lists(OM.window_lists(olay1, *cfg.window)),
                        1.0 / math.sqrt(cfg.head_dim))
    g = OL.permute(out[:, :, [h]].float().cpu().numpy(), olay1)
    real = OL.token_order(olay1) >= 0
    _gate(g[0, 0, real], O[0, 0, real], lse[0, h].cpu().numpy()[real], L[0, 0, real],
          "480p window per-tile walk head 5")


def test_topk32_bench_pipeline_every_tile_of_one_head():
    cfg = CONFIGS["topk32_16x32x32"]
    _, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    h = 7
    announce("full-size: top-32 layer through the bench's calls, head 7, all 256 tiles")
    qn, kn, vn = (to_device(x, "bf16") for x in (q, k, v))
    _, qp = vsa.tile_permute_pool(blay, qn, means_only=True)
    kt, kp = vsa.tile_permute_pool(blay, kn)
    vt = vsa.tile_permute_v(blay, vn)
    idx, cnt, _ = vsa.build_mask_topk_pooled(blay, qp, kp, top_k=cfg.top_k)
    out, lse = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, idx, cnt, want_lse=True, v_operand=True)
    torch.cuda.synchronize()
    olay1, qo = _one_head(cfg, q, h)
    _, ko = _one_head(cfg, k, h)
    _, vo = _one_head(cfg, v, h)
    sigma = 1.0 / math.sqrt(cfg.head_dim)
    s = OR.coarse_scores(OR.pool_tiles(qo, olay1), OR.pool_tiles(ko, olay1), sigma)
    ridx, rcnt = OR.select_lists_vectorized(s, top_k=cfg.top_k)
    gi, gc = idx[0, h].cpu().numpy(), cnt[0, h].cpu().numpy()
    lists = [sorted(gi[t, :gc[t]].tolist()) for t in range(olay1.n_tiles)]
    bad = [t for t in range(olay1.n_tiles)
           if not _accept_topk(lists[t], ridx[0, 0, t, :rcnt[0, 0, t]].tolist(), s[0, 0, t], cfg.top_k)]
    assert not bad, f"head {h}: {len(bad)} lists differ beyond near-ties"
    O, L = OA.attention(qo, ko, vo, olay1, OA.shared_lists(lists), sigma)
    g = OL.permute(out[:, :, [h]].float().cpu().numpy(), olay1)
    real = OL.token_order(olay1) >= 0
    _gate(g[0, 0, real], O[0, 0, real], lse[0, h].cpu().numpy()[real], L[0, 0, real],
          "top-32 bench pipeline head 7")
