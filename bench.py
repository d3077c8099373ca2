"""Benchmark: block-sparse video attention forward on one MI355X.

Default workload: the Wan-14B 768p Skiparse-2D hybrid (21x48x80 latent grid,
40 heads, d = 128, bf16): one step is one 4-layer cycle (three Skiparse-2D
sparse layers and one dense layer). Every layer runs the whole hot path from
natural-order Q, K, V to natural-order O: tile permute of K and V, attention
over the cached fixed lists (built once per shape, as a Skiparse pattern is
head- and data-invariant) with the permute of Q and the inverse permute of
O fused into the kernel. The other four workloads are measured after it and
reported under "per_workload" (one layer per step each); the routed ones
also from natural-order inputs to natural-order O: the 720p fp8 top-p layer
quantises each tensor straight from the natural order (Q and K with the
routing's tile means), routes from the means and writes O in the natural
order; the top-32 layer pools Q without a tiled copy, permutes K (with its
means) and V, and reads Q / writes O in the natural order.

Printed: ONE JSON line. value = executed TFLOP/s of the attention over the
whole timed step (permutes included in the time; ms_per_step is the median
of the per-step times, the mean is also given); roofline = the attention
kernel's executed FLOP per launch / its average launch time (HIP events on
the launch stream) against the 2.5 PFLOP/s dense bf16 peak; cpu_baseline =
the fp64 oracle timed on this host on a seeded sample of (head, query tile)
items of the sparse layer. "backward" = the sparse layer's backward pass
(dQ, dK, dV over the same lists) with its own roofline (algorithmic FLOP =
2.5x the forward's) and the gradient oracle timed the same way.
"big_tiles_480p" = attention over FPSAttention-style (6,8,8) big-tile windows
((6,6,6), (6,6,1), (3,3,1) and dense) at the 480p latent, bf16 and fp8.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                       [--only-headline] [--backward] [--no-cpu-baseline] [--calib-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0
METRIC = "sparse video-attn fwd: ms/layer, executed TFLOP/s and % of MFMA peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def exec_flops(pairs: int, d: int, tile: int) -> float:
    """Executed FLOP of attention: 4 * d * tile^2 per (query tile, key tile) pair."""
    return 4.0 * d * tile * tile * pairs


class Timer:
    """Accumulates HIP-event durations of launches on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = {}
        self.total = {}
        self.count = {}
        self.times = {}

    def run(self, name, fn):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        r = fn()
        e1.record()
        self.pending.setdefault(name, []).append((e0, e1))
        return r

    def collect(self):
        self.torch.cuda.synchronize()
        for name, evs in self.pending.items():
            for e0, e1 in evs:
                t = e0.elapsed_time(e1)
                self.total[name] = self.total.get(name, 0.0) + t
                self.count[name] = self.count.get(name, 0) + 1
                self.times.setdefault(name, []).append(t)
        self.pending.clear()

    def median(self, name):
        """Median launch time of one kernel kind (ms); robust to a stray slow launch."""
        t = sorted(self.times[name])
        m = len(t)
        return t[m // 2] if m % 2 else 0.5 * (t[m // 2 - 1] + t[m // 2])

    def reset(self):
        self.pending.clear()
        self.total.clear()
        self.count.clear()
        self.times.clear()


def to_dev(x, dtype, torch, np):
    from synth import bf16_bits
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def build_workload(name, torch, np, vsa):
    """Inputs on the GPU plus a step function for one workload."""
    from synth import CONFIGS, make_qkv
    cfg = CONFIGS[name]
    t0 = time.time()
    q, k, v = make_qkv(cfg)
    lay = vsa.Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=cfg.heads, head_dim=cfg.head_dim,
                     kind=cfg.kind, tile=cfg.tile, stride=cfg.stride)
    info = vsa.layout_info(lay)
    nat = [to_dev(x, cfg.dtype, torch, np) for x in (q, k, v)]
    del q, k, v
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s")
    C, d, n = info.tile_tokens, cfg.head_dim, info.n_tiles
    state = {"cfg": cfg, "lay": lay, "info": info}
    # bf16 layers over 64-token tiles store V in the P.V operand order, which the
    # attention kernel stages with whole 16-byte copies (same output bits)
    vop = cfg.dtype == "bf16" and C == 64

    def permute_v(x):
        return vsa.tile_permute_v(lay, x) if vop else vsa.tile_permute(lay, x)

    if cfg.mask in ("window", "skiparse"):
        radius = cfg.window if cfg.mask == "window" else (0, 0, 0)
        kv_idx, kv_cnt = vsa.build_mask_window(lay, radius)      # cached: built once per shape
        torch.cuda.synchronize()
        pairs_sparse = int(kv_cnt.sum().item()) * cfg.heads
        state["lists"] = (kv_idx, kv_cnt)

    def layer(timer, dense=False):
        if cfg.mask in ("window", "skiparse"):
            # fixed lists: Q is read and O written in the natural order by the
            # attention kernel itself; only K and V are permuted
            tk = timer.run("permute", lambda: vsa.tile_permute(lay, nat[1]))
            tv = timer.run("permute_v" if vop else "permute", lambda: permute_v(nat[2]))
            if dense:
                timer.run("attn_dense", lambda: vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, tv,
                                                                              v_operand=vop))
            else:
                # 3D windows differ between neighbouring query tiles: each tile walks its
                # own list (list_mode 2); Skiparse tiles of a group share one list and
                # walk it four at a time
                timer.run("attn", lambda: vsa.block_sparse_attn_fwd_nat(
                    lay, nat[0], tk, tv, kv_idx, kv_cnt, per_tile_walk=cfg.mask == "window",
                    v_operand=vop))
            return
        if cfg.mask == "topk":
            # routed bf16 layer: the tile means of Q come from a pass that writes no
            # tiled copy (the attention reads Q in the natural order), K is permuted
            # with its means pooled on the way, V permuted; O is written in the
            # natural order by the attention kernel
            _, qp = timer.run("pool", lambda: vsa.tile_permute_pool(lay, nat[0], means_only=True))
            tk, kp = timer.run("permute_pool", lambda: vsa.tile_permute_pool(lay, nat[1]))
            tv = timer.run("permute_v" if vop else "permute", lambda: permute_v(nat[2]))
            idx, cnt, _ = timer.run("route", lambda: vsa.build_mask_topk_pooled(
                lay, qp, kp, top_k=cfg.top_k))
            state["cnt"] = cnt
            timer.run("attn", lambda: vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, tv, idx, cnt,
                                                                    v_operand=vop))
        else:
            # fp8 top-p layer: each tensor goes from the natural order to tiled e4m3
            # codes in one pass (Q and K with the routing's tile means, V in the P.V
            # operand layout); routing on the bf16 means; the fp8 attention, dealt
            # heavy-first, writes O in the natural order
            (qc, qs, qp), (kc, ks, kp) = (timer.run("quant", lambda x=x: vsa.quant_fp8_tiles_nat(
                lay, x, want_pooled=True)) for x in nat[:2])
            vc, vs, _ = timer.run("quant", lambda: vsa.quant_fp8_tiles_nat(lay, nat[2], v_operand=True))
            idx, cnt, _ = timer.run("route", lambda: vsa.build_mask_topk_pooled(
                lay, qp, kp, top_p=cfg.top_p, k_floor=cfg.k_floor))
            state["cnt"] = cnt
            # top-p lists differ in length: deal the walks heavy-first
            order = timer.run("order", lambda: vsa.build_work_order(lay, cnt))
            timer.run("attn", lambda: vsa.block_sparse_attn_fwd_fp8_nat(
                lay, qc, kc, vc, (qs, ks, vs), idx, cnt, v_operand=True, work_order=order))

    def step(timer):
        if cfg.dense_every:
            for i in range(cfg.dense_every):
                layer(timer, dense=(i == cfg.dense_every - 1))
        else:
            layer(timer)

    def flops():
        """(executed attention FLOP per step, per attention launch kind)."""
        if cfg.mask in ("window", "skiparse"):
            sparse = exec_flops(pairs_sparse, d, C)
            if cfg.dense_every:
                dense = exec_flops(n * n * cfg.heads, d, C)
                return sparse * (cfg.dense_every - 1) + dense, {"attn": sparse, "attn_dense": dense}
            return sparse, {"attn": sparse}
        pairs = int(state["cnt"].sum().item())
        f = exec_flops(pairs, d, C)
        return f, {"attn": f}

    def dense_equiv():
        per_layer = 4.0 * d * float(info.n_tokens) ** 2 * cfg.heads
        return per_layer * (cfg.dense_every or 1)

    def head_spread():
        """Routed lists: max over heads of a head's visited pairs / the mean over heads."""
        if "cnt" not in state:
            return None
        per_head = state["cnt"].reshape(-1, cfg.heads, n).sum(dim=(0, 2)).double()
        return round(float(per_head.max() / per_head.mean()), 3)

    def cold_attn(reps=3, scratch_mb=512):
        """Sparse-layer attention with a scratch write of scratch_mb MB before each launch
        (evicts the 256 MB MALL and the L2s); returns the mean launch time in ms."""
        if cfg.mask not in ("window", "skiparse"):
            return None
        tk, tv = vsa.tile_permute(lay, nat[1]), permute_v(nat[2])
        scratch = torch.empty(scratch_mb << 20, dtype=torch.uint8, device="cuda")
        total = 0.0
        for i in range(reps):
            scratch.fill_(i + 1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            vsa.block_sparse_attn_fwd_nat(lay, nat[0], tk, tv, kv_idx, kv_cnt,
                                          per_tile_walk=cfg.mask == "window", v_operand=vop)
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        del scratch, tk, tv
        return total / reps

    def hbm_bytes():
        """Algorithmic HBM bytes per launch of each data-movement kernel: every
        input byte read once and every output byte written once (pad rows of a
        tiled tensor count as written)."""
        es = 2 if cfg.dtype == "bf16" else 4
        row = cfg.heads * d
        nat_b, til_b = info.n_tokens * row * es, info.n_padded * row * es
        means = n * row * 4
        out = {"permute": nat_b + til_b, "permute_v": nat_b + til_b, "unpermute": nat_b + til_b,
               "permute_pool": nat_b + til_b + means, "pool": nat_b + means}
        if cfg.fp8:
            codes, scales = info.n_padded * row, n * cfg.heads * 4
            # quantiser launches per layer: Q and K with their means, V without
            out["quant"] = nat_b + codes + scales + (2 * means) / 3
        return out

    state.update(step=step, flops=flops, dense_equiv=dense_equiv, nat=nat, head_spread=head_spread,
                 cold_attn=cold_attn, hbm_bytes=hbm_bytes)
    return state


def measure_backward(state, torch, vsa, steps, warmup):
    """Backward of the sparse layer: the forward's output and lse, a seeded
    upstream gradient, the transposed lists (built once per shape, like the
    fixed lists), then `steps` timed calls of the whole backward (row
    statistics, dQ and dK/dV kernels) with HIP events on the launch stream."""
    cfg, lay = state["cfg"], state["lay"]
    if cfg.mask not in ("window", "skiparse"):
        return None
    kv_idx, kv_cnt = state["lists"]
    tq, tk, tv = (vsa.tile_permute(lay, x) for x in state["nat"])
    out, lse = vsa.block_sparse_attn_fwd(lay, tq, tk, tv, kv_idx, kv_cnt, want_lse=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    dout = torch.randn(out.shape, generator=gen, device="cuda").to(out.dtype)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    q_idx, q_cnt = vsa.build_transposed_lists(lay, kv_idx, kv_cnt)
    e1.record()
    torch.cuda.synchronize()
    t_lists = e0.elapsed_time(e1)
    grads = tuple(torch.empty_like(x) for x in (tq, tk, tv))
    ws = torch.empty(vsa.bwd_workspace_bytes(lay), dtype=torch.uint8, device="cuda")

    def call():
        vsa.block_sparse_attn_bwd(lay, tq, tk, tv, out, dout, lse, kv_idx, kv_cnt, q_idx, q_cnt,
                                  grads=grads, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fwd_flops = state["flops"]()[1]["attn"]
    alg, exe = 2.5 * fwd_flops, 3.5 * fwd_flops
    del tq, tk, tv, out, lse, dout, grads, ws
    return {
        "workload": f"{cfg.name} sparse layer backward (dQ, dK, dV)",
        "ms_per_layer": round(ms, 3),
        "transposed_lists_ms": round(t_lists, 4),
        "steps": steps,
        "algorithmic_tflop": round(alg / 1e12, 3),
        "executed_tflop": round(exe / 1e12, 3),
        "executed_tflops": round(exe / (ms * 1e-3) / 1e12, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(alg / (ms * 1e-3) / 1e12, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(alg / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "traffic": bwd_traffic_from_profiles(),
        },
    }


def measure_big_tiles(torch, np, vsa, reps=5):
    """480p latent (21x30x52, 12 heads, d = 128) on (1,8,8) tiles grouped six
    along t into (6,8,8) big tiles: attention over the big-tile windows of
    the pages' ablation ((6,6,6), (6,6,1), (3,3,1)) and dense, bf16, and the
    (6,6,1) window in fp8 with one scale per big tile. Lists are built once
    per window (as a denoising-step schedule would, switching between them);
    each attention launch is timed with HIP events."""
    from synth import CONFIGS, make_qkv
    cfg = CONFIGS["window_480p"]
    q, k, v = make_qkv(cfg)
    lay = vsa.Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=cfg.heads, head_dim=cfg.head_dim,
                     tile=(1, 8, 8))
    info = vsa.layout_info(lay)
    tq, tk, tv = (vsa.tile_permute(lay, to_dev(x, "bf16", torch, np)) for x in (q, k, v))
    del q, k, v
    group = (6, 1, 1)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {"workload": "21x30x52 latent, 12 heads, d=128, (1,8,8) tiles in (6,1,1) groups = (6,8,8) big tiles",
           "windows": {}}
    dense_ms = timed(lambda: vsa.block_sparse_attn_fwd(lay, tq, tk, tv))
    n = info.n_tiles
    res["windows"]["dense"] = {"attn_ms": round(dense_ms, 4),
                               "tflops": round(exec_flops(n * n * cfg.heads, 128, 64) / (dense_ms * 1e-3) / 1e12, 2)}
    for ext in ((6, 6, 6), (6, 6, 1), (3, 3, 1)):
        idx, cnt = vsa.build_mask_window_grouped(lay, group, ext)
        pairs = int(cnt.sum().item()) * cfg.heads
        # neighbouring query tiles lie along w: with a narrow w extent their
        # lists barely overlap, so each tile walks its own list (list_mode 2);
        # a wide one keeps the union walk of four tiles
        per_tile = ext[2] < 3
        ms = timed(lambda: vsa.block_sparse_attn_fwd(lay, tq, tk, tv, idx, cnt, per_tile_walk=per_tile))
        f = exec_flops(pairs, 128, 64)
        entry = {"attn_ms": round(ms, 4), "density": round(pairs / (n * n * cfg.heads), 4),
                 "walk": "per query tile" if per_tile else "unions of four query tiles",
                 "tflops": round(f / (ms * 1e-3) / 1e12, 2),
                 "frac_of_peak": round(f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "speedup_vs_dense": round(dense_ms / ms, 3)}
        if ext == (6, 6, 1):
            (qc, qs), (kc, ks) = (vsa.quant_fp8_tiles_grouped(lay, x, group) for x in (tq, tk))
            vc, vs = vsa.quant_fp8_tiles_grouped(lay, tv, group, v_operand=True)
            qms = timed(lambda: vsa.quant_fp8_tiles_grouped(lay, tq, group))
            fms = timed(lambda: vsa.block_sparse_attn_fwd(lay, qc, kc, vc, idx, cnt, scales=(qs, ks, vs),
                                                          v_operand=True, per_tile_walk=per_tile))
            entry["fp8"] = {"attn_ms": round(fms, 4), "quant_ms_per_tensor": round(qms, 4),
                            "tflops": round(f / (fms * 1e-3) / 1e12, 2),
                            "frac_of_fp8_peak": round(f / (fms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                            "speedup_vs_dense_bf16": round(dense_ms / fms, 3)}
        res["windows"]["x".join(str(e) for e in ext)] = entry
    del tq, tk, tv
    return res


def measure(state, torch, steps, warmup):
    """Warm-up steps, then `steps` timed steps with a HIP event before each step
    and after the last (all on the launch stream). Returns the median step time
    (ms), the mean step time, the wall time of the timed region and the timer of
    the individual launches."""
    timer = Timer(torch)
    for _ in range(warmup):
        state["step"](timer)
    timer.collect()
    timer.reset()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t_wall = time.time()
    evs[0].record()
    for i in range(steps):
        state["step"](timer)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.time() - t_wall
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    median = per_step[steps // 2] if steps % 2 else 0.5 * (per_step[steps // 2 - 1] + per_step[steps // 2])
    mean = evs[0].elapsed_time(evs[-1]) / steps
    timer.collect()
    return median, mean, wall, timer


def cpu_baseline(name, np, seconds=12.0, bwd_seconds=0.0):
    """Time the fp64 oracle on a seeded sample of sparse-layer (head, query tile)
    items: the forward, and for bwd_seconds > 0 also the gradient oracle.
    Returns (forward record, backward record or None)."""
    from oracle import attention as OA
    from oracle import layout as OL
    from oracle import masks as OM
    from synth import CONFIGS, make_qkv
    cfg = CONFIGS[name]
    heads = [0, cfg.heads // 2]
    q, k, v = make_qkv(cfg)
    lay = OL.Layout(T=cfg.T, H=cfg.H, W=cfg.W, heads=len(heads), head_dim=cfg.head_dim,
                    kind=cfg.kind, tile=cfg.tile, stride=cfg.stride)
    xs = [OL.permute(np.ascontiguousarray(x[:, :, heads]), lay).astype(np.float64)
          for x in (q, k, v)]
    del q, k, v
    if cfg.mask == "skiparse":
        lists = OM.skiparse_lists(lay)
    elif cfg.mask == "window":
        lists = OM.window_lists(lay, *cfg.window)
    else:
        lists = OM.dense_lists(lay)
    rng = np.random.default_rng(1234)
    sigma = 1.0 / math.sqrt(cfg.head_dim)
    done_pairs = 0
    n_items = 0
    t0 = time.time()
    while time.time() - t0 < seconds:
        h = int(rng.integers(0, len(heads)))
        t = int(rng.integers(0, lay.n_tiles))
        OA.attention(*xs, lay, OA.shared_lists(lists), sigma, items=[(0, h, t)])
        done_pairs += len(lists[t])
        n_items += 1
    el = time.time() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in blas] + [1])
        blas_name = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or "unknown"
    except Exception:
        threads, blas_name = len(os.sched_getaffinity(0)), "unknown"
    fwd = {
        "value": exec_flops(done_pairs, cfg.head_dim, lay.tile_tokens) / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "blas": blas_name,
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{n_items} seeded (head, query-tile) items of the {name} sparse layer, "
                  f"fp64 numpy, {el:.1f}s wall",
    }
    if bwd_seconds <= 0:
        return fwd, None
    # the gradient oracle on the same items' kind: one query tile's share of dQ, dK, dV
    from oracle import attention_grad as OG
    g = rng.standard_normal(xs[0].shape)
    done_pairs = n_items = 0
    t0 = time.time()
    while time.time() - t0 < bwd_seconds:
        h = int(rng.integers(0, len(heads)))
        t = int(rng.integers(0, lay.n_tiles))
        OG.attention_backward(*xs, g, lay, OA.shared_lists(lists), sigma, items=[(0, h, t)])
        done_pairs += len(lists[t])
        n_items += 1
    el = time.time() - t0
    bwd = {
        "value": 2.5 * exec_flops(done_pairs, cfg.head_dim, lay.tile_tokens) / el / 1e12,
        "unit": "TFLOP/s (algorithmic: 2.5x the forward's FLOP)",
        "cores": int(threads),
        "blas": blas_name,
        "kind": "oracle",
        "sample": f"{n_items} seeded (head, query-tile) items of the {name} sparse layer backward, "
                  f"fp64 numpy, {el:.1f}s wall",
    }
    return fwd, bwd


def code_hash(path):
    """sha256 of a source file's code: comments, trailing blanks and empty
    lines removed, so that a comment edit does not invalidate counters taken
    on the same code."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [ln.rstrip() for ln in text.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def traffic_from_profiles(kernel_src_hash):
    """HBM bytes per attention launch from the committed counter summary.

    The summary records the code hash (code_hash) of the attention source it
    was measured on; if the kernel's code has changed since, the figure is
    stale and None is returned.
    """
    path = os.path.join(ROOT, "profiles", "attn_skiparse_768p_pmc.md")
    rec = {}
    try:
        with open(path) as f:
            for line in f:
                if ":" in line and line.split(":", 1)[0] in ("attn_code_sha256", "bytes_per_launch"):
                    k, v = line.split(":", 1)
                    rec[k] = v.strip()
    except OSError:
        return None
    if rec.get("attn_code_sha256") != kernel_src_hash or "bytes_per_launch" not in rec:
        return None
    return int(rec["bytes_per_launch"])


def bwd_traffic_from_profiles():
    """HBM bytes per backward call (row statistics, dQ and dK/dV kernels) from
    the committed counter summary, or None if the backward source changed."""
    path = os.path.join(ROOT, "profiles", "attn_bwd_skiparse_768p_pmc.md")
    sha = code_hash(os.path.join(ROOT, "block_sparse_attention_token_amd", "csrc", "attn_bwd.hip"))
    rec = {}
    try:
        with open(path) as f:
            for line in f:
                if ":" in line and line.split(":", 1)[0] in ("bwd_code_sha256", "bytes_per_call"):
                    k, v = line.split(":", 1)
                    rec[k] = v.strip()
    except OSError:
        return None
    if rec.get("bwd_code_sha256") != sha or "bytes_per_call" not in rec:
        return None
    return int(rec["bytes_per_call"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="skiparse_768p")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mall-cold", action="store_true",
                    help="skip the attention launches timed after a 512 MB scratch write")
    ap.add_argument("--backward", action="store_true",
                    help="time the sparse-layer backward also with --only-headline")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also launch one plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the block-sparse attention path on "
              "one GPU (no multi-GPU mode); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_token_amd as vsa
    torch.cuda.init()

    if args.calib_copy:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)   # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 1 GiB read + 1 GiB written")

    head = build_workload(args.workload, torch, np, vsa)
    cfg = head["cfg"]
    ms_step, ms_mean, wall, timer = measure(head, torch, args.steps, args.warmup)
    step_flops, per_launch = head["flops"]()
    value = step_flops / (ms_step * 1e-3) / 1e12
    layers = cfg.dense_every or 1
    # roofline: the attention kernel over every attention launch of the timed steps
    attn_ms = sum(timer.total.get(k, 0.0) for k in ("attn", "attn_dense"))
    attn_n = sum(timer.count.get(k, 0) for k in ("attn", "attn_dense"))
    attn_flops = sum(per_launch[k] * timer.count.get(k, 0) for k in per_launch)
    peak = FP8_PEAK_TFLOPS if cfg.fp8 else BF16_PEAK_TFLOPS
    achieved = (attn_flops / attn_n) / (attn_ms / attn_n * 1e-3) / 1e12
    src_hash = code_hash(os.path.join(ROOT, "block_sparse_attention_token_amd", "csrc", "attn.hip"))
    kernels = {k: {"ms_avg": timer.total[k] / timer.count[k], "launches_per_step": timer.count[k] // args.steps}
               for k in timer.total}
    for k, f in per_launch.items():
        if k in kernels:
            kernels[k]["tflops"] = f / (kernels[k]["ms_avg"] * 1e-3) / 1e12
            kernels[k]["frac_of_peak"] = kernels[k]["tflops"] / peak
    cold_ms = None if args.no_mall_cold else head["cold_attn"]()
    if cold_ms is not None:
        kernels["attn_mall_cold"] = {
            "ms_avg": cold_ms, "note": "sparse layer, 512 MB scratch write before each launch",
            "tflops": per_launch["attn"] / (cold_ms * 1e-3) / 1e12,
            "frac_of_peak": per_launch["attn"] / (cold_ms * 1e-3) / 1e12 / peak}
    info = head["info"]
    hbm = head["hbm_bytes"]()
    for k in hbm:
        if k in kernels:
            kernels[k]["gbs"] = hbm[k] / (kernels[k]["ms_avg"] * 1e-3) / 1e9
            kernels[k]["frac_of_hbm_peak"] = kernels[k]["gbs"] / HBM_PEAK_GBS
    # plain device-to-device copy of 1 GiB on the same device: the HBM rate a
    # pure read + write stream reaches here (reference for the permute's rate)
    src_c = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    dst_c = torch.empty_like(src_c)
    dst_c.copy_(src_c)
    torch.cuda.synchronize()
    ec0, ec1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ec0.record()
    for _ in range(5):
        dst_c.copy_(src_c)
    ec1.record()
    torch.cuda.synchronize()
    kernels["copy_1GiB_reference"] = {"gbs": 2 * (1 << 30) * 5 / (ec0.elapsed_time(ec1) * 1e-3) / 1e9}
    del src_c, dst_c

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "ms_per_step_mean": round(ms_mean, 3),
        "timing": "median of the per-step HIP-event times (mean also given)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if cfg.fp8 else cfg.dtype,
        "data": "synthetic (seeded Q/K/V of the workload's shape and distribution)",
        "config": {
            "workload": cfg.name,
            "grid_thw": [cfg.T, cfg.H, cfg.W],
            "heads": cfg.heads,
            "head_dim": cfg.head_dim,
            "tile": list(cfg.tile),
            "mask": cfg.mask,
            "dense_every": cfg.dense_every,
            "layers_per_step": layers,
            "ms_per_layer": round(ms_step / layers, 3),
            "exec_tflop_per_step": round(step_flops / 1e12, 3),
            "frac_of_mfma_peak": round(value / peak, 4),
            "dense_equiv_tflops": round(head["dense_equiv"]() / (ms_step * 1e-3) / 1e12, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            # the committed counters are of the 768p Skiparse step's attention launches
            "traffic": traffic_from_profiles(src_hash) if args.workload == "skiparse_768p" else None,
        },
        "kernels": kernels,
        "wall_s_timed": round(wall, 2),
    }
    if not args.only_headline or args.backward:
        log("timing the sparse layer backward")
        out["backward"] = measure_backward(head, torch, vsa, args.steps, args.warmup)
    del head
    torch.cuda.empty_cache()

    if not args.only_headline:
        from synth import CONFIGS
        per = {}
        for name in CONFIGS:
            if name == args.workload:
                continue
            st = build_workload(name, torch, np, vsa)
            ms, _, _, tm = measure(st, torch, 20, 3)
            f, pl = st["flops"]()
            pk = FP8_PEAK_TFLOPS if st["cfg"].fp8 else BF16_PEAK_TFLOPS
            a_ms = tm.median("attn")
            per[name] = {
                "ms_per_layer": round(ms / (st["cfg"].dense_every or 1), 4),
                "exec_tflops_step": round(f / (ms * 1e-3) / 1e12, 2),
                "attn_ms": round(a_ms, 4),
                "attn_tflops": round(pl["attn"] / (a_ms * 1e-3) / 1e12, 2),
                "attn_frac_of_peak": round(pl["attn"] / (a_ms * 1e-3) / 1e12 / pk, 4),
                "peak_tflops": pk,
                "kernels_ms": {k: round(tm.median(k), 4) for k in tm.total},
                "kernel_times": "median launch time per kernel kind",
            }
            hbm = st["hbm_bytes"]()
            per[name]["hbm"] = {k: {"gb_per_launch": round(hbm[k] / 1e9, 4),
                                    "gbs": round(hbm[k] / (tm.median(k) * 1e-3) / 1e9, 1),
                                    "frac_of_hbm_peak": round(hbm[k] / (tm.median(k) * 1e-3)
                                                              / 1e9 / HBM_PEAK_GBS, 4)}
                                for k in hbm if k in tm.total}
            if st["cfg"].fp8:
                per[name]["attn_frac_of_bf16_peak"] = round(
                    pl["attn"] / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
            spread = st["head_spread"]()
            if spread is not None:
                per[name]["head_pairs_max_over_mean"] = spread
            log(f"{name}: {per[name]}")
            del st
            torch.cuda.empty_cache()
        out["per_workload"] = per
        log("timing big-tile windows")
        out["big_tiles_480p"] = measure_big_tiles(torch, np, vsa)
        log(f"big tiles: {out['big_tiles_480p']}")

    if not args.no_cpu_baseline:
        log("timing the oracle on host cores")
        fwd, bwd = cpu_baseline(args.workload, np,
                                bwd_seconds=0.0 if args.only_headline else 6.0)
        out["cpu_baseline"] = fwd
        if bwd is not None and out.get("backward"):
            out["backward"]["cpu_baseline"] = bwd
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
