"""GPU parity: block-sparse attention forward against the fp64 oracle.

Both sides get identical key-tile lists: the oracle's lists are uploaded to
the GPU. Gates: bf16 max-abs 2e-2 and relative L2 1e-2. fp8: relative L2
5e-2 against the oracle of the fp8 method (oracle e4m3 quantiser, then fp64
attention on the dequantised tensors); against the oracle on the unquantised
bf16 inputs the kernel may add at most 10% (+5e-3) to the error the
quantisation itself causes there.
LSE: 2e-3 absolute for bf16 inputs; for fp32 inputs, which the kernel rounds
to bf16, up to 2.5e-2 (bound: sigma * 2 * 2^-9 * sum_e |q_e k_e|, about 0.024
at d = 64 with unit-variance inputs).
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
from tests.gpu_util import (announce, errors, inputs, layouts, lists_to_device, table_from_lists,
                            to_device)

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2, REL_L2_FP8 = 2e-2, 1e-2, 5e-2
# fp8 lse gates. One-tile (routed) walk: the row sum adds the unrounded
# weights in fp32, so lse follows the dequantised oracle up to fp32 rounding
# of scores and exp2. Four-tile walks sum the e4m3-rounded weights on the
# matrix core: each weight in the e4m3 normal range is off by at most 2^-4
# relatively (half an e4m3 step), so the row sum is off by at most 2^-4 and
# lse by at most ln(1 + 2^-4) = 0.061 (measured: up to 3.5e-2 on rows whose
# list is one or two tiles, where a few weights dominate); gate 6.5e-2.
FP8_LSE_GATE = {"routed": 2e-3, "window_union": 6.5e-2, "shared_lengths": 6.5e-2}


def _tiled(cfg, olay, blay, x):
    return vsa.tile_permute(blay, to_device(x, cfg.dtype)), OL.permute(x, olay).astype(np.float64)


def _items(olay, n, seed, must=()):
    rng = np.random.default_rng(seed)
    picks = {(0, int(h), int(t)) for h, t in zip(rng.integers(0, olay.heads, n),
                                                  rng.integers(0, olay.n_tiles, n))}
    picks |= set(must)
    return sorted(picks)


def _compare(out_gpu, O_ref, lse_gpu, L_ref, olay, items, rel_gate=REL_L2, abs_gate=MAX_ABS,
             lse_gate=2e-3):
    C = olay.tile_tokens
    g, r, gl, rl = [], [], [], []
    for b, h, t in items:
        g.append(out_gpu[b, h, t * C:(t + 1) * C])
        r.append(O_ref[b, h, t * C:(t + 1) * C])
        if lse_gpu is not None:
            gl.append(lse_gpu[b, h, t * C:(t + 1) * C])
            rl.append(L_ref[b, h, t * C:(t + 1) * C])
    g, r = np.concatenate(g), np.concatenate(r)
    mae, rl2 = errors(g, r)
    print(f"max_abs={mae:.3e} rel_l2={rl2:.3e}")
    assert mae <= abs_gate and rl2 <= rel_gate, (mae, rl2)
    if gl:
        gl, rl = np.concatenate(gl), np.concatenate(rl)
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.abs(gl[fin] - rl[fin]).max() <= lse_gate
    return mae, rl2


def _run_shared(name, radius, n_items, dense=False, seed=0, full=False, per_tile=False):
    cfg = CONFIGS[name]
    olay, blay = layouts(cfg)
    q, k, v = inputs(name)
    sigma = 1.0 / math.sqrt(cfg.head_dim)
    lists = OM.dense_lists(olay) if dense else OM.window_lists(olay, *radius)
    idx, cnt = table_from_lists(lists)
    announce(f"attn {name} radius={radius} dense={dense}")
    qd, qo = _tiled(cfg, olay, blay, q)
    kd, ko = _tiled(cfg, olay, blay, k)
    vd, vo = _tiled(cfg, olay, blay, v)
    if dense:
        out, lse = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, want_lse=True)
    else:
        di, dc = lists_to_device(idx, cnt)
        out, lse = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc, want_lse=True,
                                             per_tile_walk=per_tile)
    torch.cuda.synchronize()
    items = None if full else _items(olay, n_items, seed,
                                     must=[(0, 0, 0), (0, olay.heads - 1, olay.n_tiles - 1)])
    O, L = OA.attention(qo, ko, vo, olay, OA.shared_lists(lists), sigma, items=items)
    if items is None:
        items = [(0, h, t) for h in range(olay.heads) for t in range(olay.n_tiles)]
    _compare(out.float().cpu().numpy(), O, lse.cpu().numpy(), L, olay, items,
             lse_gate=2.5e-2 if cfg.dtype == "f32" else 2e-3)
    return out


def test_tiny_f32_full():
    _run_shared("tiny_window_f32", (1, 1, 1), 0, full=True)


def test_window_480p_sampled():
    _run_shared("window_480p", (1, 2, 2), 150, seed=3)


def test_window_480p_per_tile_walk_sampled():
    """The launch bench.py times for the 480p window workload: the shared
    table walked per query tile (list_mode 2)."""
    _run_shared("window_480p", (1, 2, 2), 150, seed=13, per_tile=True)


def test_skiparse_768p_sparse_sampled():
    _run_shared("skiparse_768p", (0, 0, 0), 24, seed=4)


def test_skiparse_768p_dense_layer_sampled():
    _run_shared("skiparse_768p", (0, 0, 0), 10, dense=True, seed=5)


def _routed(name, top_k=0, top_p=0.0, k_floor=0):
    cfg = CONFIGS[name]
    olay, _ = layouts(cfg)
    q, k, _ = inputs(name)
    qb = OR.pool_tiles(OL.permute(q, olay), olay)
    kb = OR.pool_tiles(OL.permute(k, olay), olay)
    s = OR.coarse_scores(qb, kb, 1.0 / math.sqrt(cfg.head_dim))
    return OR.select_lists_vectorized(s, top_k=top_k, top_p=top_p, k_floor=k_floor)


def test_topk32_full():
    cfg = CONFIGS["topk32_16x32x32"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    idx, cnt = _routed(cfg.name, top_k=cfg.top_k)
    idx = np.ascontiguousarray(idx[..., :cfg.top_k])
    announce(f"attn {cfg.name} routed top-k")
    qd, qo = _tiled(cfg, olay, blay, q)
    kd, ko = _tiled(cfg, olay, blay, k)
    vd, vo = _tiled(cfg, olay, blay, v)
    di, dc = lists_to_device(idx, cnt)
    out, lse = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc, want_lse=True)
    torch.cuda.synchronize()
    lists_fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    O, L = OA.attention(qo, ko, vo, olay, lists_fn, 1.0 / math.sqrt(cfg.head_dim))
    items = [(0, h, t) for h in range(olay.heads) for t in range(olay.n_tiles)]
    _compare(out.float().cpu().numpy(), O, lse.cpu().numpy(), L, olay, items)
    # determinism: a second launch is bit-identical
    out2, _ = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.fixture(scope="module")
def topp_case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cfg = CONFIGS["fp8_topp_720p"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    idx, cnt = _routed(cfg.name, top_p=cfg.top_p, k_floor=cfg.k_floor)
    qd, qo = _tiled(cfg, olay, blay, q)
    kd, ko = _tiled(cfg, olay, blay, k)
    vd, vo = _tiled(cfg, olay, blay, v)
    return cfg, olay, blay, idx, cnt, (qd, kd, vd), (qo, ko, vo)


def test_topp_720p_fp8_sampled(topp_case):
    cfg, olay, blay, idx, cnt, (qd, kd, vd), (qo, ko, vo) = topp_case
    announce(f"attn {cfg.name} fp8 routed top-p")
    qc, qs = vsa.quant_fp8_tiles(blay, qd)
    kc, ks = vsa.quant_fp8_tiles(blay, kd)
    vc, vs = vsa.quant_fp8_tiles(blay, vd)
    di, dc = lists_to_device(idx, cnt)
    out, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, di, dc, scales=(qs, ks, vs))
    torch.cuda.synchronize()
    og = out.float().cpu().numpy()
    # oracle side on 4 heads (quantisation is independent per head)
    rng = np.random.default_rng(6)
    heads = sorted(rng.choice(cfg.heads, 4, replace=False).tolist())
    sub = OL.Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=4, head_dim=cfg.head_dim, tile=cfg.tile)
    xs = [x[:, heads].astype(np.float32) for x in (qo, ko, vo)]
    deq = [OF.dequantize_tiles(*OF.quantize_tiles(x, sub), sub) for x in xs]
    items = [(0, j, int(t)) for j in range(4) for t in rng.integers(0, olay.n_tiles, 5)]
    items.append((0, 3, olay.n_tiles - 1))
    lists_fn = lambda b, j, t: idx[b, heads[j], t, :cnt[b, heads[j], t]].tolist()
    sigma = 1.0 / math.sqrt(cfg.head_dim)
    Od, _ = OA.attention(*deq, sub, lists_fn, sigma, items=items)
    Ou, _ = OA.attention(*(x.astype(np.float64) for x in xs), sub, lists_fn, sigma, items=items)
    C = olay.tile_tokens
    g = np.concatenate([og[0, heads[j], t * C:(t + 1) * C] for _, j, t in items])
    rd = np.concatenate([Od[0, j, t * C:(t + 1) * C] for _, j, t in items])
    ru = np.concatenate([Ou[0, j, t * C:(t + 1) * C] for _, j, t in items])
    mae_d, rl2_d = errors(g, rd)
    mae_u, rl2_u = errors(g, ru)
    _, rl2_q = errors(rd, ru)
    print(f"fp8 vs oracle(dequantised): max_abs={mae_d:.3e} rel_l2={rl2_d:.3e}; "
          f"vs oracle(bf16): rel_l2={rl2_u:.3e}; quantisation alone: rel_l2={rl2_q:.3e}")
    assert rl2_d <= REL_L2_FP8
    assert rl2_u <= 1.1 * rl2_q + 5e-3


def test_topp_720p_fp8_v_operand_identical(topp_case):
    """V codes in the P.V operand layout give the very same output as the
    token-major codes (same arithmetic, only the staging differs)."""
    cfg, olay, blay, idx, cnt, (qd, kd, vd), _ = topp_case
    announce(f"attn {cfg.name} fp8 v-operand")
    qc, qs = vsa.quant_fp8_tiles(blay, qd)
    kc, ks = vsa.quant_fp8_tiles(blay, kd)
    vc, vs = vsa.quant_fp8_tiles(blay, vd)
    vo, vs2 = vsa.quant_fp8_tiles(blay, vd, v_operand=True)
    di, dc = lists_to_device(idx, cnt)
    o1, l1 = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, di, dc, scales=(qs, ks, vs), want_lse=True)
    o2, l2 = vsa.block_sparse_attn_fwd(blay, qc, kc, vo, di, dc, scales=(qs, ks, vs2), want_lse=True,
                                       v_operand=True)
    # shared lists too (the grouped kernel)
    sh = OM.window_lists(olay, 1, 1, 1)
    si, sc = lists_to_device(*table_from_lists(sh))
    o3, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, si, sc, scales=(qs, ks, vs))
    o4, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vo, si, sc, scales=(qs, ks, vs2), v_operand=True)
    torch.cuda.synchronize()
    assert torch.equal(vs, vs2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(o3.view(torch.int16), o4.view(torch.int16))


def test_topp_720p_bf16_sampled(topp_case):
    cfg, olay, blay, idx, cnt, (qd, kd, vd), (qo, ko, vo) = topp_case
    announce(f"attn {cfg.name} bf16 routed top-p")
    di, dc = lists_to_device(idx, cnt)
    out, lse = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc, want_lse=True)
    torch.cuda.synchronize()
    items = _items(olay, 16, 7, must=[(0, olay.heads - 1, olay.n_tiles - 1)])
    lists_fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    O, L = OA.attention(qo, ko, vo, olay, lists_fn, 1.0 / math.sqrt(cfg.head_dim), items=items)
    _compare(out.float().cpu().numpy(), O, lse.cpu().numpy(), L, olay, items)


def test_empty_lists_pad_rows_and_guard_band():
    cfg = CONFIGS["window_480p"]
    olay, blay = layouts(cfg, heads=2)
    rng = np.random.default_rng(9)
    from synth import round_to_bf16
    q, k, v = (round_to_bf16(rng.standard_normal((1, olay.n_tokens, 2, 128)).astype(np.float32))
               for _ in range(3))
    lists = OM.window_lists(olay, 0, 1, 1)
    lists = [[] if t % 7 == 3 else row for t, row in enumerate(lists)]   # some empty lists
    idx, cnt = table_from_lists(lists, width=9)
    announce("attn empty lists + guard band")
    qd, qo = _tiled(cfg, olay, blay, q)
    kd, ko = _tiled(cfg, olay, blay, k)
    vd, vo = _tiled(cfg, olay, blay, v)
    di, dc = lists_to_device(idx, cnt)
    n = olay.n_padded * 2 * 128
    guard = 4096
    buf = torch.full((n + guard,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = buf[:n].view(1, 2, olay.n_padded, 128)
    vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc, out=out)
    torch.cuda.synchronize()
    assert bool((buf[n:] == 3.0).all())
    O, _ = OA.attention(qo, ko, vo, olay, OA.shared_lists(lists), 1.0 / math.sqrt(128))
    og = out.float().cpu().numpy()
    C = olay.tile_tokens
    for t in range(olay.n_tiles):
        if t % 7 == 3:
            assert np.all(og[0, :, t * C:(t + 1) * C] == 0)
    order = OL.token_order(olay)
    assert np.all(og[0, :, order < 0] == 0)
    items = [(0, h, t) for h in range(2) for t in range(olay.n_tiles)]
    _compare(og, O, None, None, olay, items)


def test_list_modes_agree():
    """A shared table and the same table repeated per head give the same output.

    The two list modes run different kernels (four query tiles per workgroup
    over 64-token kv tiles vs. one query tile over 32-token kv blocks), which
    round P to bf16 at different points, so agreement is to bf16 rounding."""
    cfg = CONFIGS["window_480p"]
    olay, blay = layouts(cfg, heads=3)
    rng = np.random.default_rng(10)
    from synth import round_to_bf16
    x = [round_to_bf16(rng.standard_normal((1, olay.n_tokens, 3, 128)).astype(np.float32))
         for _ in range(3)]
    lists = OM.window_lists(olay, 1, 1, 1)
    idx, cnt = table_from_lists(lists)
    announce("attn list modes")
    t = [vsa.tile_permute(blay, to_device(a, "bf16")) for a in x]
    di, dc = lists_to_device(idx, cnt)
    o1, _ = vsa.block_sparse_attn_fwd(blay, *t, di, dc)
    di4 = di[None, None].expand(1, 3, *di.shape).contiguous()
    dc4 = dc[None, None].expand(1, 3, *dc.shape).contiguous()
    o2, _ = vsa.block_sparse_attn_fwd(blay, *t, di4, dc4)
    torch.cuda.synchronize()
    mae, rl2 = errors(o1.float().cpu().numpy(), o2.float().cpu().numpy().astype(np.float64))
    assert mae <= 1e-2 and rl2 <= 5e-3


def test_shared_walk_list_lengths():
    """Every list length from 1 to 9, and a few past the buffer ring, on the
    walk taken when a workgroup's four query tiles share one list.

    Groups of four consecutive query tiles get one list of random key tiles
    (some of them padded at the grid's edge); the group's length cycles
    through 1..9, 13..17, so the walk ends at every position of its unrolled
    loop and at every phase of its buffer ring."""
    cfg = CONFIGS["window_480p"]
    olay, blay = layouts(cfg, heads=2)
    rng = np.random.default_rng(12)
    from synth import round_to_bf16
    q, k, v = (round_to_bf16(rng.standard_normal((1, olay.n_tokens, 2, 128)).astype(np.float32))
               for _ in range(3))
    lengths = [1, 2, 3, 4, 5, 6, 7, 8, 9, 13, 14, 15, 16, 17]
    lists = []
    for g in range((olay.n_tiles + 3) // 4):
        n = lengths[g % len(lengths)]
        row = sorted(rng.choice(olay.n_tiles, n, replace=False).tolist())
        lists += [row] * 4
    lists = lists[:olay.n_tiles]
    idx, cnt = table_from_lists(lists)
    announce("attn shared walk, list lengths 1..17")
    qd, qo = _tiled(cfg, olay, blay, q)
    kd, ko = _tiled(cfg, olay, blay, k)
    vd, vo = _tiled(cfg, olay, blay, v)
    di, dc = lists_to_device(idx, cnt)
    out, lse = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc, want_lse=True)
    torch.cuda.synchronize()
    # one query tile of every group whose length is below 18, both heads
    items = [(0, h, 4 * g + (g % 4)) for g in range(len(lengths) * 2) for h in range(2)]
    items = [it for it in items if it[2] < olay.n_tiles]
    O, L = OA.attention(qo, ko, vo, olay, OA.shared_lists(lists), 1.0 / math.sqrt(128), items=items)
    _compare(out.float().cpu().numpy(), O, lse.cpu().numpy(), L, olay, items)


@pytest.mark.parametrize("tile,d,dtype", [((4, 4, 4), 64, "bf16"), ((2, 4, 4), 128, "bf16"),
                                          ((2, 4, 4), 64, "bf16"), ((4, 4, 4), 128, "f32"),
                                          ((4, 4, 4), 64, "f32"), ((2, 4, 4), 128, "f32")])
@pytest.mark.parametrize("mode", ["shared", "routed"])
def test_tile_and_head_dim_shapes(tile, d, dtype, mode):
    """Every tile size / head size / input type the kernels take, on a ragged
    grid, with shared window lists (query tiles walking one union) and with
    routed per-head lists of random length (empty lists included)."""
    T, H, W, heads = 7, 10, 13, 2
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile)
    rng = np.random.default_rng(1200 + 100 * tile[0] + d + 7 * (dtype == "f32") + 3 * (mode == "routed"))
    from synth import round_to_bf16
    q, k, v = (rng.standard_normal((1, olay.n_tokens, heads, d)).astype(np.float32) for _ in range(3))
    if dtype == "bf16":
        q, k, v = (round_to_bf16(x) for x in (q, k, v))
    announce(f"attn shapes tile={tile} d={d} {dtype} {mode}")
    qd, qo = (vsa.tile_permute(blay, to_device(q, dtype)), OL.permute(q, olay).astype(np.float64))
    kd, ko = (vsa.tile_permute(blay, to_device(k, dtype)), OL.permute(k, olay).astype(np.float64))
    vd, vo = (vsa.tile_permute(blay, to_device(v, dtype)), OL.permute(v, olay).astype(np.float64))
    n = olay.n_tiles
    if mode == "shared":     # one list per group of four query tiles: the pipelined walk
        lists = []
        for g in range((n + 3) // 4):
            row = sorted(set(rng.choice(n, 8, replace=False).tolist()) | {0, 3, 5})
            lists += [row] * 4
        lists = lists[:n]
        idx, cnt = table_from_lists(lists)
        lists_fn = OA.shared_lists(lists)
    else:
        width = max(1, n // 2)
        idx = np.full((1, heads, n, width), -1, dtype=np.int32)
        cnt = np.zeros((1, heads, n), dtype=np.int32)
        for h in range(heads):
            for t in range(n):
                c = int(rng.integers(0, width + 1))
                idx[0, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                cnt[0, h, t] = c
        lists_fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    di, dc = lists_to_device(idx, cnt)
    out, lse = vsa.block_sparse_attn_fwd(blay, qd, kd, vd, di, dc, want_lse=True)
    torch.cuda.synchronize()
    O, Lr = OA.attention(qo, ko, vo, olay, lists_fn, 1.0 / math.sqrt(d))
    items = [(0, h, t) for h in range(heads) for t in range(n)]
    # fp32 inputs are rounded to bf16 for the products: the lse bound grows with d
    _compare(out.float().cpu().numpy(), O, lse.cpu().numpy(), Lr, olay, items,
             lse_gate=(2.5e-2 if d == 64 else 5e-2) if dtype == "f32" else 2e-3)


@pytest.mark.parametrize("mode", ["window_union", "shared_lengths", "routed"])
def test_fp8_walks(mode):
    """fp8 attention on every walk: unions of window lists (plain walk), one
    list per group of four query tiles with lengths 1..9 and 13..17
    (pipelined walk ending at every position), and routed per-head lists with
    empty ones; gated against the oracle of the fp8 method."""
    T, H, W, heads, d = 9, 14, 22, 2, 128
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(4, 4, 4))
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(4, 4, 4))
    rng = np.random.default_rng({"window_union": 1301, "shared_lengths": 1302, "routed": 1303}[mode])
    from synth import round_to_bf16
    x = [round_to_bf16(rng.standard_normal((1, olay.n_tokens, heads, d)).astype(np.float32))
         for _ in range(3)]
    announce(f"attn fp8 {mode}")
    n = olay.n_tiles
    if mode == "window_union":
        lists = OM.window_lists(olay, 1, 1, 1)
    elif mode == "shared_lengths":
        lengths = [1, 2, 3, 4, 5, 6, 7, 8, 9, 13, 14, 15, 16, 17]
        lists = []
        for g in range((n + 3) // 4):
            row = sorted(rng.choice(n, min(lengths[g % len(lengths)], n), replace=False).tolist())
            lists += [row] * 4
        lists = lists[:n]
    if mode == "routed":
        width = n // 2
        idx = np.full((1, heads, n, width), -1, dtype=np.int32)
        cnt = np.zeros((1, heads, n), dtype=np.int32)
        for h in range(heads):
            for t in range(n):
                c = int(rng.integers(0, width + 1))
                idx[0, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                cnt[0, h, t] = c
        lists_fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    else:
        idx, cnt = table_from_lists(lists)
        lists_fn = OA.shared_lists(lists)
    tiled = [vsa.tile_permute(blay, to_device(a, "bf16")) for a in x]
    (qc, qs), (kc, ks), (vc, vs) = (vsa.quant_fp8_tiles(blay, t) for t in tiled)
    di, dc = lists_to_device(idx, cnt)
    out, lse = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, di, dc, scales=(qs, ks, vs), want_lse=True)
    torch.cuda.synchronize()
    xo = [OL.permute(a, olay).astype(np.float32) for a in x]
    deq = [OF.dequantize_tiles(*OF.quantize_tiles(a, olay), olay) for a in xo]
    O, Lr = OA.attention(*deq, olay, lists_fn, 1.0 / math.sqrt(d))
    og = out.float().cpu().numpy()
    C = olay.tile_tokens
    items = [(0, h, t) for h in range(heads) for t in range(n)]
    g = np.concatenate([og[0, h, t * C:(t + 1) * C] for _, h, t in items])
    r = np.concatenate([O[0, h, t * C:(t + 1) * C] for _, h, t in items])
    mae, rl2 = errors(g, r)
    # lse against the oracle's on the dequantised inputs (natural log)
    lg, lr = lse.cpu().numpy(), Lr
    fin = np.isfinite(lr)
    assert np.array_equal(np.isfinite(lg), fin)
    lerr = float(np.abs(lg[fin] - lr[fin]).max())
    print(f"fp8 {mode}: max_abs={mae:.3e} rel_l2={rl2:.3e} lse_max_abs={lerr:.3e}")
    assert rl2 <= REL_L2_FP8
    assert lerr <= FP8_LSE_GATE[mode]
    empty = [(h, t) for h in range(heads) for t in range(n) if not lists_fn(0, h, t)]
    for h, t in empty:
        assert np.all(og[0, h, t * C:(t + 1) * C] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["shared", "routed"])
@pytest.mark.parametrize("scale", [0.17, -0.3, 0.0])
def test_batch_and_softmax_scales(dtype, mode, scale):
    """Batch of two, a softmax scale other than 1/sqrt(d), a negative one
    (folded into Q) and zero (uniform weights over the key set)."""
    T, H, W, heads, d, B = 5, 9, 10, 2, 128, 2
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(4, 4, 4), batch=B)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(4, 4, 4), batch=B)
    rng = np.random.default_rng(1400 + int(1000 * scale) + 10 * (mode == "routed") + (dtype == "fp8"))
    from synth import round_to_bf16
    x = [round_to_bf16(rng.standard_normal((B, olay.n_tokens, heads, d)).astype(np.float32))
         for _ in range(3)]
    announce(f"attn batch 2 scale {scale} {mode} {dtype}")
    n = olay.n_tiles
    if mode == "shared":
        lists = OM.window_lists(olay, 1, 1, 1)
        idx, cnt = table_from_lists(lists)
        lists_fn = OA.shared_lists(lists)
    else:
        width = max(1, n // 2)
        idx = np.full((B, heads, n, width), -1, dtype=np.int32)
        cnt = np.zeros((B, heads, n), dtype=np.int32)
        for b in range(B):
            for h in range(heads):
                for t in range(n):
                    c = int(rng.integers(1, width + 1))
                    idx[b, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                    cnt[b, h, t] = c
        lists_fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    tiled = [vsa.tile_permute(blay, to_device(a, "bf16")) for a in x]
    xo = [OL.permute(a, olay).astype(np.float64) for a in x]
    di, dc = lists_to_device(idx, cnt)
    if dtype == "fp8":
        (qc, qs), (kc, ks), (vc, vs) = (vsa.quant_fp8_tiles(blay, t) for t in tiled)
        out, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, di, dc, softmax_scale=scale,
                                           scales=(qs, ks, vs))
        xo = [OF.dequantize_tiles(*OF.quantize_tiles(a.astype(np.float32), olay), olay) for a in xo]
    else:
        out, _ = vsa.block_sparse_attn_fwd(blay, *tiled, di, dc, softmax_scale=scale)
    torch.cuda.synchronize()
    O, _ = OA.attention(*xo, olay, lists_fn, scale)
    og = out.float().cpu().numpy()
    mae, rl2 = errors(og, np.nan_to_num(O))
    print(f"scale {scale} {mode} {dtype}: max_abs={mae:.3e} rel_l2={rl2:.3e}")
    if dtype == "fp8":
        assert rl2 <= REL_L2_FP8
    else:
        assert mae <= MAX_ABS and rl2 <= REL_L2


@pytest.mark.parametrize("kind,tile,d,dtype,mode", [
    ("tile3d", (4, 4, 4), 128, "bf16", "shared"), ("tile3d", (4, 4, 4), 64, "f32", "routed"),
    ("tile3d", (2, 4, 4), 128, "bf16", "dense"), ("tile3d", (4, 4, 4), 128, "bf16", "per_tile"),
    ("skiparse2d", (4, 4, 4), 128, "bf16", "shared")])
def test_natural_io_forward(kind, tile, d, dtype, mode):
    """Q read and O written in the natural order inside the kernel: the output
    is bit-identical to the tiled forward followed by the inverse permute, and
    matches the oracle; batch 2, ragged grids (and Skiparse group tails)."""
    T, H, W, heads, B = (5, 9, 13, 2, 2) if kind == "tile3d" else (3, 10, 12, 2, 2)
    kw = dict(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile, kind=kind, stride=(2, 2))
    olay, blay = OL.Layout(**kw, batch=B), vsa.Layout(**kw, batch=B)
    rng = np.random.default_rng(3300 + d + len(mode) + (kind == "skiparse2d"))
    xs = [rng.standard_normal((B, olay.n_tokens, heads, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        from synth import round_to_bf16
        xs = [round_to_bf16(x) for x in xs]
    announce(f"natural io {kind} tile={tile} d={d} {dtype} {mode}")
    qn, kn, vn = (to_device(x, dtype) for x in xs)
    qt, kt, vt = (vsa.tile_permute(blay, x) for x in (qn, kn, vn))
    n = olay.n_tiles
    if mode in ("shared", "per_tile"):
        lists = OM.skiparse_lists(olay) if kind == "skiparse2d" else OM.window_lists(olay, 1, 1, 1)
        idx, cnt = table_from_lists(lists)
        fn = OA.shared_lists(lists)
    elif mode == "routed":
        width = max(1, n // 2)
        idx = np.full((B, heads, n, width), -1, dtype=np.int32)
        cnt = np.zeros((B, heads, n), dtype=np.int32)
        for b in range(B):
            for h in range(heads):
                for t in range(n):
                    c = int(rng.integers(0, width + 1))
                    idx[b, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                    cnt[b, h, t] = c
        fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    else:
        idx = cnt = None
        fn = OA.shared_lists(OM.dense_lists(olay))
    di, dc = lists_to_device(idx, cnt) if idx is not None else (None, None)
    pt = mode == "per_tile"
    out_t, lse_t = vsa.block_sparse_attn_fwd(blay, qt, kt, vt, di, dc, want_lse=True, per_tile_walk=pt)
    ref_nat = vsa.tile_permute(blay, out_t, inverse=True)
    out_n, lse_n = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, di, dc, want_lse=True, per_tile_walk=pt)
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int16) if dtype == "bf16" else out_n.view(torch.int32),
                       ref_nat.view(torch.int16) if dtype == "bf16" else ref_nat.view(torch.int32))
    assert torch.equal(lse_n, lse_t)
    O, _ = OA.attention(*(OL.permute(x, olay).astype(np.float64) for x in xs), olay, fn, 1.0 / math.sqrt(d))
    mae, rl2 = errors(out_n.float().cpu().numpy(), OL.unpermute(O, olay))
    assert mae <= 2e-2 and rl2 <= 1e-2, (mae, rl2)


def test_natural_io_skiparse_768p_identical():
    """The launch bench.py times for the 768p Skiparse sparse layer: natural
    Q in, natural O out, bit-identical to the tiled forward + inverse permute."""
    cfg = CONFIGS["skiparse_768p"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    announce("natural io skiparse 768p")
    qn, kn, vn = (to_device(x, cfg.dtype) for x in (q, k, v))
    qt, kt, vt = (vsa.tile_permute(blay, x) for x in (qn, kn, vn))
    idx, cnt = vsa.build_mask_window(blay, (0, 0, 0))
    out_t, _ = vsa.block_sparse_attn_fwd(blay, qt, kt, vt, idx, cnt)
    ref = vsa.tile_permute(blay, out_t, inverse=True)
    out_n, _ = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt, idx, cnt)
    dense_t, _ = vsa.block_sparse_attn_fwd(blay, qt, kt, vt)
    dense_ref = vsa.tile_permute(blay, dense_t, inverse=True)
    dense_n, _ = vsa.block_sparse_attn_fwd_nat(blay, qn, kt, vt)
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(dense_n.view(torch.int16), dense_ref.view(torch.int16))


@pytest.mark.parametrize("mode", ["shared", "routed"])
@pytest.mark.parametrize("vop", [False, True])
def test_fp8_zero_tiles(mode, vop):
    """Tiles whose absmax is 0 (scale 0, all codes 0) in Q, K and V: a zero K
    tile scores 0, a zero Q tile gives uniform weights over its key set, a
    zero V tile keeps its softmax weight but adds nothing to O; both walks
    (the four-tile walk sums P on the matrix core) and both V layouts, gated
    against the oracle of the fp8 method."""
    T, H, W, heads, d = 6, 10, 14, 2, 128
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(4, 4, 4))
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(4, 4, 4))
    rng = np.random.default_rng(1401 + 2 * vop + (mode == "routed"))
    from synth import round_to_bf16
    x = [round_to_bf16(rng.standard_normal((1, olay.n_tokens, heads, d)).astype(np.float32))
         for _ in range(3)]
    order = OL.token_order(olay)
    C, n = olay.tile_tokens, olay.n_tiles
    for which, tiles in ((0, (1, n - 2)), (1, (0, 3, n - 1)), (2, (2, 5, n - 3))):
        for t in tiles:
            nat = order[t * C:(t + 1) * C]
            x[which][0, nat[nat >= 0], t % heads, :] = 0.0
    announce(f"attn fp8 zero tiles {mode} v_operand={vop}")
    if mode == "shared":
        lists = OM.window_lists(olay, 1, 1, 1)
        idx, cnt = table_from_lists(lists)
        lists_fn = OA.shared_lists(lists)
    else:
        width = n // 2
        idx = np.full((1, heads, n, width), -1, dtype=np.int32)
        cnt = np.zeros((1, heads, n), dtype=np.int32)
        for h in range(heads):
            for t in range(n):
                row = sorted(set(rng.choice(n, width - 1, replace=False).tolist()) | {0, 3, 5})[:width]
                idx[0, h, t, :len(row)] = row
                cnt[0, h, t] = len(row)
        lists_fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    tiled = [vsa.tile_permute(blay, to_device(a, "bf16")) for a in x]
    (qc, qs), (kc, ks) = (vsa.quant_fp8_tiles(blay, t) for t in tiled[:2])
    vc, vs = vsa.quant_fp8_tiles(blay, tiled[2], v_operand=vop)
    di, dc = lists_to_device(idx, cnt)
    out, _ = vsa.block_sparse_attn_fwd(blay, qc, kc, vc, di, dc, scales=(qs, ks, vs), v_operand=vop)
    torch.cuda.synchronize()
    assert int((qs == 0).sum()) == 2 and int((ks == 0).sum()) == 3 and int((vs == 0).sum()) == 3
    xo = [OL.permute(a, olay).astype(np.float32) for a in x]
    deq = [OF.dequantize_tiles(*OF.quantize_tiles(a, olay), olay) for a in xo]
    O, _ = OA.attention(*deq, olay, lists_fn, 1.0 / math.sqrt(d))
    og = out.float().cpu().numpy()
    assert np.all(np.isfinite(og))
    items = [(0, h, t) for h in range(heads) for t in range(n)]
    g = np.concatenate([og[0, h, t * C:(t + 1) * C] for _, h, t in items])
    r = np.concatenate([O[0, h, t * C:(t + 1) * C] for _, h, t in items])
    mae, rl2 = errors(g, r)
    print(f"fp8 zero tiles {mode} vop={vop}: max_abs={mae:.3e} rel_l2={rl2:.3e}")
    assert rl2 <= REL_L2_FP8
