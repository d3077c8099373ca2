"""GPU parity: gradients of the block-sparse attention against the fp64 oracle.

Both sides get identical key-tile lists (the oracle's lists are uploaded) and
identical seeded inputs and upstream gradients. The GPU backward runs on the
GPU forward's own output and lse, as a training step would.

Gates (per gradient, over the rows compared): relative L2 <= 1e-2 and
max-abs <= 2e-2 * max|reference| for bf16 inputs; fp32 inputs, which the
kernels round to bf16 for the products exactly as the forward does, get
relative L2 <= 2e-2 and max-abs <= 4e-2 * max|reference|. The bf16 budget
covers the operands the kernels round to bf16 (P and dS before their
products, 2^-9 relative each), the bf16 output O inside D = dO . O and the
bf16 rounding of the gradients themselves; the fp32-input budget adds the
rounding of Q, K, V and dO, which moves scores by up to
sigma * 2^-8 * sum_e |q_e k_e| (the bound the forward's lse gate uses).
Transposed lists are integer work: bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from oracle import attention as OA
from oracle import attention_grad as OG
from oracle import layout as OL
from oracle import masks as OM
from oracle import routing as OR
from synth import CONFIGS, make_grad, round_to_bf16
from tests.gpu_util import announce, errors, inputs, layouts, lists_to_device, table_from_lists, to_device

pytestmark = pytest.mark.gpu

GATES = {"bf16": (1e-2, 2e-2), "f32": (2e-2, 4e-2)}


def _check(name, gpu, ref, dtype):
    rel_gate, abs_gate = GATES[dtype]
    mae, rl2 = errors(gpu, ref)
    scale = float(np.abs(ref).max())
    print(f"{name}: max_abs={mae:.3e} (max|ref|={scale:.3e}) rel_l2={rl2:.3e}")
    assert rl2 <= rel_gate and mae <= abs_gate * max(scale, 1e-30), (name, mae, scale, rl2)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


class Case:
    """Tiled inputs on both sides, GPU forward, GPU backward."""

    def __init__(self, olay, blay, q, k, v, g, dtype, lists_fn, idx=None, cnt=None, sigma=None):
        self.olay, self.blay, self.dtype = olay, blay, dtype
        self.sigma = 1.0 / math.sqrt(olay.head_dim) if sigma is None else sigma
        self.lists_fn = lists_fn
        dev = [vsa.tile_permute(blay, to_device(x, dtype)) for x in (q, k, v, g)]
        self.qd, self.kd, self.vd, self.gd = dev
        self.qo, self.ko, self.vo, self.go = (OL.permute(x, olay).astype(np.float64)
                                              for x in (q, k, v, g))
        if idx is not None:
            self.di, self.dc = lists_to_device(idx, cnt)
        else:
            self.di = self.dc = None
        self.out, self.lse = vsa.block_sparse_attn_fwd(blay, self.qd, self.kd, self.vd, self.di,
                                                       self.dc, softmax_scale=self.sigma,
                                                       want_lse=True)
        self.grads = vsa.block_sparse_attn_bwd(blay, self.qd, self.kd, self.vd, self.out, self.gd,
                                               self.lse, self.di, self.dc, softmax_scale=self.sigma)
        torch.cuda.synchronize()

    def compare_full(self):
        ref = OG.attention_backward(self.qo, self.ko, self.vo, self.go, self.olay, self.lists_fn,
                                    self.sigma)
        for nm, gpu, r in zip(("dq", "dk", "dv"), self.grads, ref):
            _check(nm, _np(gpu), r, self.dtype)
        return ref


def _rand_routed(olay, B, rng, width, allow_empty=True):
    n = olay.n_tiles
    idx = np.full((B, olay.heads, n, width), -1, dtype=np.int32)
    cnt = np.zeros((B, olay.heads, n), dtype=np.int32)
    for b in range(B):
        for h in range(olay.heads):
            for t in range(n):
                c = int(rng.integers(0 if allow_empty else 1, width + 1))
                idx[b, h, t, :c] = np.sort(rng.choice(n, c, replace=False))
                cnt[b, h, t] = c
    return idx, cnt, (lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist())


def _small_inputs(olay, B, dtype, rng, std=1.0):
    shape = (B, olay.n_tokens, olay.heads, olay.head_dim)
    xs = [rng.standard_normal(shape).astype(np.float32) * np.float32(s)
          for s in (std, std, 1.0, 1.0)]
    return [round_to_bf16(x) for x in xs] if dtype == "bf16" else xs


# ---------------------------------------------------------------------------
def test_transposed_lists_bitexact():
    """Shared window table, per-(b, head) random lists with empty rows, and
    Skiparse group lists: every row equals the oracle's transposition."""
    announce("bwd transposed lists")
    olay, blay = layouts(CONFIGS["window_480p"], heads=2)
    table = OM.window_lists(olay, 1, 2, 2)
    idx, cnt = table_from_lists(table)
    di, dc = lists_to_device(idx, cnt)
    qi, qc = vsa.build_transposed_lists(blay, di, dc)
    ref = OG.transposed_lists(olay, OA.shared_lists(table), 1)[0][0]
    qi, qc = qi.cpu().numpy(), qc.cpu().numpy()
    for j in range(olay.n_tiles):
        assert qc[j] == len(ref[j]) and qi[j, :qc[j]].tolist() == ref[j]
    # routed
    rng = np.random.default_rng(31)
    idx, cnt, fn = _rand_routed(olay, 2, rng, 40)
    di, dc = lists_to_device(idx, cnt)
    blay2 = vsa.Layout(T=olay.T, H=olay.H, W=olay.W, heads=2, head_dim=128, batch=2)
    qi, qc = vsa.build_transposed_lists(blay2, di, dc)
    ref = OG.transposed_lists(olay, fn, 2)
    qi, qc = qi.cpu().numpy(), qc.cpu().numpy()
    for b in range(2):
        for h in range(2):
            for j in range(olay.n_tiles):
                r = ref[b][h][j]
                assert qc[b, h, j] == len(r) and qi[b, h, j, :len(r)].tolist() == r
    # skiparse 768p groups: every key tile is held by the 315 tiles of its group
    solay, sblay = layouts(CONFIGS["skiparse_768p"], heads=1)
    table = OM.skiparse_lists(solay)
    idx, cnt = table_from_lists(table)
    di, dc = lists_to_device(idx, cnt)
    qi, qc = vsa.build_transposed_lists(sblay, di, dc)
    qi, qc = qi.cpu().numpy(), qc.cpu().numpy()
    for j in range(solay.n_tiles):
        assert qi[j, :qc[j]].tolist() == table[j]


def test_tiny_f32_full():
    """The 4x8x8 fp32 workload (32-token tiles, d = 64), all rows."""
    cfg = CONFIGS["tiny_window_f32"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    g = make_grad(cfg)
    lists = OM.window_lists(olay, *cfg.window)
    idx, cnt = table_from_lists(lists)
    announce("bwd tiny f32")
    Case(olay, blay, q, k, v, g, "f32", OA.shared_lists(lists), idx, cnt).compare_full()


@pytest.mark.parametrize("tile,d,dtype", [((4, 4, 4), 128, "bf16"), ((4, 4, 4), 64, "bf16"),
                                          ((2, 4, 4), 128, "bf16"), ((2, 4, 4), 64, "bf16"),
                                          ((4, 4, 4), 128, "f32"), ((2, 4, 4), 64, "f32")])
@pytest.mark.parametrize("mode", ["shared", "routed", "dense"])
def test_shapes_and_list_modes(tile, d, dtype, mode):
    """Every tile size / head size / input type, on a ragged grid (pad rows in
    query and key tiles), with a shared window table, routed per-(b, head)
    random lists with empty rows (batch 2), and dense attention."""
    T, H, W, heads = 5, 9, 13, 2
    B = 2 if mode == "routed" else 1
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=tile, batch=B)
    rng = np.random.default_rng(2100 + 10 * tile[0] + d + 3 * (dtype == "f32") + len(mode))
    q, k, v, g = _small_inputs(olay, B, dtype, rng)
    announce(f"bwd shapes tile={tile} d={d} {dtype} {mode}")
    if mode == "shared":
        lists = OM.window_lists(olay, 1, 1, 1)
        idx, cnt = table_from_lists(lists)
        fn = OA.shared_lists(lists)
    elif mode == "routed":
        idx, cnt, fn = _rand_routed(olay, B, rng, max(1, olay.n_tiles // 2))
    else:
        idx = cnt = None
        fn = OA.shared_lists(OM.dense_lists(olay))
    Case(olay, blay, q, k, v, g, dtype, fn, idx, cnt).compare_full()


def test_skiparse_group_tails():
    """Skiparse-2D with a padded tail tile in every residue group."""
    T, H, W, heads, d = 3, 10, 12, 2, 128
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind="skiparse2d", stride=(2, 2))
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind="skiparse2d", stride=(2, 2))
    assert olay.group_len % olay.tile_tokens != 0
    rng = np.random.default_rng(2301)
    q, k, v, g = _small_inputs(olay, 1, "bf16", rng)
    lists = OM.skiparse_lists(olay)
    idx, cnt = table_from_lists(lists)
    announce("bwd skiparse tails")
    Case(olay, blay, q, k, v, g, "bf16", OA.shared_lists(lists), idx, cnt).compare_full()


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.17])
def test_softmax_scales(scale):
    """Zero scale (uniform weights: dQ = dK = 0), a negative scale and a small one."""
    T, H, W, heads, d = 4, 8, 12, 2, 128
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d)
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d)
    rng = np.random.default_rng(2400 + int(100 * abs(scale)))
    q, k, v, g = _small_inputs(olay, 1, "bf16", rng)
    idx, cnt, fn = _rand_routed(olay, 1, rng, olay.n_tiles // 2)
    announce(f"bwd softmax scale {scale}")
    c = Case(olay, blay, q, k, v, g, "bf16", fn, idx, cnt, sigma=scale)
    if scale == 0.0:
        assert float(c.grads[0].abs().max()) == 0.0 and float(c.grads[1].abs().max()) == 0.0
        ref = OG.attention_backward(c.qo, c.ko, c.vo, c.go, olay, fn, 0.0)
        _check("dv", _np(c.grads[2]), ref[2], "bf16")
    else:
        c.compare_full()


def test_topk32_full_and_deterministic():
    """The 16x32x32 top-32 routed workload (12 heads, d = 128), every row, and
    a second call bit-identical to the first."""
    cfg = CONFIGS["topk32_16x32x32"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    g = make_grad(cfg)
    qb = OR.pool_tiles(OL.permute(q, olay), olay)
    kb = OR.pool_tiles(OL.permute(k, olay), olay)
    s = OR.coarse_scores(qb, kb, 1.0 / math.sqrt(cfg.head_dim))
    idx, cnt = OR.select_lists_vectorized(s, top_k=cfg.top_k)
    idx = np.ascontiguousarray(idx[..., :cfg.top_k])
    fn = lambda b, h, t: idx[b, h, t, :cnt[b, h, t]].tolist()
    announce("bwd topk32 full")
    c = Case(olay, blay, q, k, v, g, "bf16", fn, idx, cnt)
    c.compare_full()
    again = vsa.block_sparse_attn_bwd(blay, c.qd, c.kd, c.vd, c.out, c.gd, c.lse, c.di, c.dc)
    torch.cuda.synchronize()
    for a, b in zip(c.grads, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_skiparse_768p_sampled():
    """The 768p Skiparse sparse layer at full size (40 heads, 1,260 tiles):
    dQ of sampled query tiles and dK / dV of sampled key tiles against the
    oracle, and over every head the conservation laws sum_j dK_j = 0 and
    sum_j dV_j = sum_i dO_i, which hold at any size."""
    cfg = CONFIGS["skiparse_768p"]
    olay, blay = layouts(cfg)
    q, k, v = inputs(cfg.name)
    g = make_grad(cfg)
    lists = OM.skiparse_lists(olay)
    idx, cnt = table_from_lists(lists)
    fn = OA.shared_lists(lists)
    announce("bwd skiparse 768p sampled")
    c = Case(olay, blay, q, k, v, g, "bf16", fn, idx, cnt)
    dq, dk, dv = (x.float() for x in c.grads)
    C = olay.tile_tokens
    rng = np.random.default_rng(2501)
    q_items = [(0, int(h), int(t)) for h, t in zip(rng.integers(0, olay.heads, 6),
                                                   rng.integers(0, olay.n_tiles, 6))]
    q_items += [(0, 0, 0), (0, olay.heads - 1, olay.n_tiles - 1)]
    ref_dq, _, _ = OG.attention_backward(c.qo, c.ko, c.vo, c.go, olay, fn, c.sigma, items=q_items)
    gq = np.concatenate([_np(dq[0, h, t * C:(t + 1) * C]) for _, h, t in q_items])
    rq = np.concatenate([ref_dq[0, h, t * C:(t + 1) * C] for _, h, t in q_items])
    _check("dq sampled", gq, rq, "bf16")
    gk, gv, rk, rv = [], [], [], []
    for h, kt in ((3, 17), (olay.heads - 1, olay.n_tiles - 1)):
        qts = [t for t in range(olay.n_tiles) if kt in lists[t]]
        dk_r, dv_r = OG.key_tile_gradients(c.qo, c.ko, c.vo, c.go, olay, fn, c.sigma, 0, h, kt,
                                           query_tiles=qts)
        gk.append(_np(dk[0, h, kt * C:(kt + 1) * C]))
        gv.append(_np(dv[0, h, kt * C:(kt + 1) * C]))
        rk.append(dk_r)
        rv.append(dv_r)
    _check("dk sampled", np.concatenate(gk), np.concatenate(rk), "bf16")
    _check("dv sampled", np.concatenate(gv), np.concatenate(rv), "bf16")
    # conservation laws over all heads (every 768p row is real and every list non-empty)
    sum_dk = dk[0].double().sum(dim=1)                    # [heads, d]
    tot_dk = dk[0].double().abs().sum(dim=1)
    assert float((sum_dk.abs() / tot_dk).max()) < 2e-2
    sum_dv = dv[0].double().sum(dim=1)
    sum_do = c.gd[0].double().sum(dim=1)
    rel = (sum_dv - sum_do).norm() / sum_do.norm()
    print(f"sum dV vs sum dO rel={float(rel):.3e}")
    assert float(rel) < 1e-2


def test_more_than_4096_tiles():
    """A grid of 4,352 query tiles (past the 4,096-tile limit of the grouped
    walks): the forward and the dQ kernel walk per tile, the transposed lists
    cover every key tile; sampled rows against the oracle."""
    T, H, W, heads, d = 34, 64, 64, 1, 64
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(2, 4, 4))
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, tile=(2, 4, 4))
    assert olay.n_tiles == 4352
    rng = np.random.default_rng(3101)
    q, k, v, g = _small_inputs(olay, 1, "bf16", rng)
    announce("bwd 4352 tiles")
    # a shared table of random ascending lists (the lists are inputs here;
    # the mask builders are tested on their own)
    n = olay.n_tiles
    lists = [sorted(rng.choice(n, int(rng.integers(1, 12)), replace=False).tolist()) for _ in range(n)]
    lists[0] = [0, 5, 4350]
    idx, cnt = table_from_lists(lists)
    c = Case(olay, blay, q, k, v, g, "bf16", OA.shared_lists(lists), idx, cnt)
    C = olay.tile_tokens
    items = [(0, 0, t) for t in (0, 1, 2177, 4351)]
    O, _ = OA.attention(c.qo, c.ko, c.vo, olay, OA.shared_lists(lists), c.sigma, items=items)
    go = np.concatenate([_np(c.out[0, 0, t * C:(t + 1) * C]) for _, _, t in items])
    ro = np.concatenate([O[0, 0, t * C:(t + 1) * C] for _, _, t in items])
    mae, rl2 = errors(go, ro)
    assert mae <= 2e-2 and rl2 <= 1e-2
    dq_r, _, _ = OG.attention_backward(c.qo, c.ko, c.vo, c.go, olay, OA.shared_lists(lists), c.sigma,
                                       items=items)
    _check("dq sampled", np.concatenate([_np(c.grads[0][0, 0, t * C:(t + 1) * C]) for _, _, t in items]),
           np.concatenate([dq_r[0, 0, t * C:(t + 1) * C] for _, _, t in items]), "bf16")
    for kt in (5, 4350):
        qts = [t for t in range(n) if kt in lists[t]]
        assert qts
        dk_r, dv_r = OG.key_tile_gradients(c.qo, c.ko, c.vo, c.go, olay, OA.shared_lists(lists), c.sigma,
                                           0, 0, kt, query_tiles=qts)
        _check("dk sampled", _np(c.grads[1][0, 0, kt * C:(kt + 1) * C]), dk_r, "bf16")
        _check("dv sampled", _np(c.grads[2][0, 0, kt * C:(kt + 1) * C]), dv_r, "bf16")


def test_workgroup_shapes_bit_identical():
    """LDS race check: one Skiparse table passed once (the dQ kernel runs four
    query tiles per workgroup, eight waves sharing staged K/V blocks) and
    repeated per head (one query tile per workgroup, two waves). Tiles of a
    residue group share their list, so every wave does the same products in
    the same order either way: dQ, dK and dV must be bit-identical."""
    T, H, W, heads, d = 5, 12, 20, 3, 128
    olay = OL.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind="skiparse2d", stride=(2, 2))
    blay = vsa.Layout(T=T, H=H, W=W, heads=heads, head_dim=d, kind="skiparse2d", stride=(2, 2))
    rng = np.random.default_rng(2701)
    q, k, v, g = _small_inputs(olay, 1, "bf16", rng)
    idx, cnt = table_from_lists(OM.skiparse_lists(olay))
    announce("bwd workgroup shapes bit-identical")
    c = Case(olay, blay, q, k, v, g, "bf16", None, idx, cnt)
    di4 = c.di[None, None].expand(1, heads, *c.di.shape).contiguous()
    dc4 = c.dc[None, None].expand(1, heads, *c.dc.shape).contiguous()
    per_head = vsa.block_sparse_attn_bwd(blay, c.qd, c.kd, c.vd, c.out, c.gd, c.lse, di4, dc4,
                                         softmax_scale=c.sigma)
    torch.cuda.synchronize()
    for nm, a, b in zip(("dq", "dk", "dv"), c.grads, per_head):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
