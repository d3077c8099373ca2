"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/vsa.h, derives layouts, and rejects bad arguments before
any launch (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_token_amd as vsa
from block_sparse_attention_token_amd import _lib as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)          # aligned, never dereferenced: every call below fails validation


def _declared():
    text = open(os.path.join(ROOT, "include", "vsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared()
    assert len(names) >= 10
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED)


def test_version_and_status_strings():
    L = B.lib()
    assert L.vsa_version().decode().count(".") == 2
    assert L.vsa_status_string(0) == b"VSA_OK"
    assert L.vsa_status_string(3) == b"VSA_ERR_WORKSPACE"


@pytest.mark.parametrize("T,H,W,tile,kind,npad,ntiles", [
    (4, 8, 8, (2, 4, 4), "tile3d", 256, 8),
    (21, 30, 52, (4, 4, 4), "tile3d", 39936, 624),
    (21, 48, 80, (4, 4, 4), "skiparse2d", 80640, 1260),
    (21, 45, 80, (4, 4, 4), "tile3d", 92160, 1440),
    (3, 4, 6, (1, 4, 4), "skiparse2d", 128, 8),
])
def test_layout_query(T, H, W, tile, kind, npad, ntiles):
    info = vsa.layout_info(vsa.Layout(T=T, H=H, W=W, heads=2, head_dim=64, tile=tile, kind=kind))
    assert (info.n_padded, info.n_tiles, info.n_tokens) == (npad, ntiles, T * H * W)


def _status(fn, *args):
    return getattr(B.lib(), fn)(*args)


def test_invalid_layouts():
    for lay in (vsa.Layout(T=0, H=8, W=8, heads=1, head_dim=64),
                vsa.Layout(T=4, H=8, W=8, heads=0, head_dim=64),
                vsa.Layout(T=4, H=7, W=8, heads=1, head_dim=64, kind="skiparse2d")):
        info = B.VsaLayoutInfo()
        c = lay.c()
        assert _status("vsa_layout_query", ctypes.byref(c), ctypes.byref(info)) == B.VSA_ERR_INVALID
        assert B.lib().vsa_last_error() != b""
    assert _status("vsa_layout_query", None, ctypes.byref(B.VsaLayoutInfo())) == B.VSA_ERR_INVALID


def test_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=128).c()
    L = ctypes.byref(lay)
    # permute: null pointers, unsupported dtype, misaligned pointer
    assert _status("vsa_tile_permute", L, B.VSA_BF16, None, FAKE, 0, None) == B.VSA_ERR_INVALID
    assert _status("vsa_tile_permute", L, B.VSA_FP8_E4M3, FAKE, FAKE, 0, None) == B.VSA_ERR_UNSUPPORTED
    assert _status("vsa_tile_permute", L, B.VSA_BF16, ctypes.c_void_p(0x100008), FAKE, 0, None) \
        == B.VSA_ERR_INVALID
    # window mask: max_kv below the longest list (75)
    assert _status("vsa_build_mask_window", L, 1, 2, 2, 74, FAKE, FAKE, None) == B.VSA_ERR_INVALID
    # routing: missing workspace, bad top_k, too-small max_kv
    assert _status("vsa_build_mask_topk", L, FAKE, FAKE, ctypes.c_float(0.1), 32,
                   ctypes.c_float(0.0), 0, 32, FAKE, FAKE, None, None, 0, None) == B.VSA_ERR_WORKSPACE
    assert _status("vsa_build_mask_topk", L, FAKE, FAKE, ctypes.c_float(0.1), 0,
                   ctypes.c_float(0.0), 0, 32, FAKE, FAKE, None, FAKE, 1 << 40, None) == B.VSA_ERR_INVALID
    assert _status("vsa_build_mask_topk", L, FAKE, FAKE, ctypes.c_float(0.1), 0,
                   ctypes.c_float(0.9), 16, 600, FAKE, FAKE, None, FAKE, 1 << 40, None) == B.VSA_ERR_INVALID
    # attention: one list pointer without the other, bad list_mode, fp8 without scales,
    # unsupported head_dim / tile size
    args = [FAKE, FAKE, FAKE, None, None, None]
    assert _status("vsa_block_sparse_attn_fwd", L, B.VSA_BF16, *args, FAKE, None, 8, 0,
                   None, ctypes.c_float(0.1), FAKE, None, None) == B.VSA_ERR_INVALID
    assert _status("vsa_block_sparse_attn_fwd", L, B.VSA_BF16, *args, FAKE, FAKE, 8, 3,
                   None, ctypes.c_float(0.1), FAKE, None, None) == B.VSA_ERR_INVALID
    assert _status("vsa_block_sparse_attn_fwd", L, B.VSA_FP8_E4M3, *args, FAKE, FAKE, 8, 0,
                   None, ctypes.c_float(0.1), FAKE, None, None) == B.VSA_ERR_INVALID
    assert _status("vsa_block_sparse_attn_fwd", L, B.VSA_BF16, *args, FAKE, FAKE, 8, 0,
                   None, ctypes.c_float(float("nan")), FAKE, None, None) == B.VSA_ERR_INVALID
    lay96 = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=96).c()
    assert _status("vsa_block_sparse_attn_fwd", ctypes.byref(lay96), B.VSA_BF16, *args, None, None,
                   0, 0, None, ctypes.c_float(0.1), FAKE, None, None) == B.VSA_ERR_UNSUPPORTED
    lay27 = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=128, tile=(3, 3, 3)).c()
    assert _status("vsa_block_sparse_attn_fwd", ctypes.byref(lay27), B.VSA_BF16, *args, None, None,
                   0, 0, None, ctypes.c_float(0.1), FAKE, None, None) == B.VSA_ERR_UNSUPPORTED
    # quantiser: null scales
    assert _status("vsa_quant_fp8_tiles", L, FAKE, FAKE, None, None) == B.VSA_ERR_INVALID


def test_workspace_query():
    lay = vsa.Layout(T=21, H=45, W=80, heads=40, head_dim=128).c()
    n = B.lib().vsa_build_mask_topk_workspace(ctypes.byref(lay))
    # the pooled means of Q and K only: no n_tiles x n_tiles score buffer
    assert n == 2 * 40 * 1440 * 128 * 4
    bad = vsa.Layout(T=0, H=45, W=80, heads=40, head_dim=128).c()
    assert B.lib().vsa_build_mask_topk_workspace(ctypes.byref(bad)) == 0


def _fake(i):
    """Distinct aligned fake device addresses (never dereferenced)."""
    return ctypes.c_void_p(0x100000 + 0x1000 * i)


def test_backward_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=128).c()
    L = ctypes.byref(lay)
    ws = B.lib().vsa_block_sparse_attn_bwd_workspace(L)
    assert ws == 2 * 24 * 32 * 52 * 8
    q, k, v, o, do, lse, dq, dk, dv, w = (_fake(i) for i in range(10))
    ok_tail = [ctypes.c_float(0.1), dq, dk, dv, w, ws, None]

    def bwd(dtype=B.VSA_BF16, lists=(None, None, 0, None, None), mode=0, tail=None, lay_ref=L,
            ptrs=None):
        p = ptrs or (q, k, v, o, do, lse)
        return _status("vsa_block_sparse_attn_bwd", lay_ref, dtype, *p, *lists, mode,
                       *(tail or ok_tail))

    # missing lse, partial lists, bad list_mode, fp8 dtype, NaN scale
    assert bwd(ptrs=(q, k, v, o, do, None)) == B.VSA_ERR_INVALID
    assert bwd(lists=(_fake(20), _fake(21), 8, None, None)) == B.VSA_ERR_INVALID
    assert bwd(lists=(_fake(20), _fake(21), 8, _fake(22), _fake(23)), mode=2) == B.VSA_ERR_INVALID
    assert bwd(dtype=B.VSA_FP8_E4M3) == B.VSA_ERR_UNSUPPORTED
    assert bwd(tail=[ctypes.c_float(float("nan")), dq, dk, dv, w, ws, None]) == B.VSA_ERR_INVALID
    # gradients aliasing inputs or each other, misaligned pointer
    assert bwd(tail=[ctypes.c_float(0.1), q, dk, dv, w, ws, None]) == B.VSA_ERR_INVALID
    assert bwd(tail=[ctypes.c_float(0.1), dq, dq, dv, w, ws, None]) == B.VSA_ERR_INVALID
    assert bwd(ptrs=(ctypes.c_void_p(0x100008), k, v, o, do, lse)) == B.VSA_ERR_INVALID
    # workspace missing / too small / misaligned
    assert bwd(tail=[ctypes.c_float(0.1), dq, dk, dv, None, ws, None]) == B.VSA_ERR_WORKSPACE
    assert bwd(tail=[ctypes.c_float(0.1), dq, dk, dv, w, ws - 1, None]) == B.VSA_ERR_WORKSPACE
    assert bwd(tail=[ctypes.c_float(0.1), dq, dk, dv, ctypes.c_void_p(0x100004), ws, None]) \
        == B.VSA_ERR_INVALID
    # unsupported head_dim
    lay96 = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=96).c()
    assert bwd(lay_ref=ctypes.byref(lay96)) == B.VSA_ERR_UNSUPPORTED
    # transposed lists: null outputs, bad max_kv, bad list_mode
    tl = "vsa_build_transposed_lists"
    assert _status(tl, L, _fake(20), _fake(21), 8, 0, None, _fake(22), None) == B.VSA_ERR_INVALID
    assert _status(tl, L, _fake(20), _fake(21), 0, 0, _fake(22), _fake(23), None) == B.VSA_ERR_INVALID
    assert _status(tl, L, _fake(20), _fake(21), 8, 3, _fake(22), _fake(23), None) == B.VSA_ERR_INVALID


def test_big_tile_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=128, tile=(1, 8, 8)).c()
    L = ctypes.byref(lay)
    g = "vsa_build_mask_window_grouped"
    # (6,1,1) groups of (1,8,8) tiles, extents (6,6,1): the longest list is 4*4*1 groups
    # = 21 frames (all 4 groups along t) * 4 rows * 1 column
    assert _status(g, L, 6, 1, 1, 6, 6, 1, 83, _fake(1), _fake(2), None) == B.VSA_ERR_INVALID
    assert _status(g, L, 6, 1, 1, 6, 6, 0, 84, _fake(1), _fake(2), None) == B.VSA_ERR_INVALID
    assert _status(g, L, 0, 1, 1, 6, 6, 1, 84, _fake(1), _fake(2), None) == B.VSA_ERR_INVALID
    assert _status(g, L, 6, 1, 1, 6, 6, 1, 84, None, _fake(2), None) == B.VSA_ERR_INVALID
    sk = vsa.Layout(T=21, H=48, W=80, heads=2, head_dim=128, kind="skiparse2d").c()
    assert _status(g, ctypes.byref(sk), 1, 1, 1, 1, 1, 1, 315, _fake(1), _fake(2), None) \
        == B.VSA_ERR_UNSUPPORTED
    q = "vsa_quant_fp8_tiles_grouped"
    assert _status(q, L, 6, 0, 1, _fake(1), _fake(2), _fake(3), 0, None) == B.VSA_ERR_INVALID
    assert _status(q, L, 6, 1, 1, None, _fake(2), _fake(3), 0, None) == B.VSA_ERR_INVALID
    assert _status(q, L, 6, 1, 1, _fake(1), ctypes.c_void_p(0x100008), _fake(3), 1, None) \
        == B.VSA_ERR_INVALID
    assert _status(q, ctypes.byref(sk), 1, 1, 1, _fake(1), _fake(2), _fake(3), 0, None) \
        == B.VSA_ERR_UNSUPPORTED


def test_natural_forward_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=128).c()
    L = ctypes.byref(lay)
    f = "vsa_block_sparse_attn_fwd_nat"
    q, k, v, o = (_fake(i) for i in range(4))
    # fp8 codes cannot be read in the natural order; null q; bad list_mode; NaN scale
    assert _status(f, L, B.VSA_FP8_E4M3, q, k, v, None, None, 0, 0, None, ctypes.c_float(0.1), o, None,
                   None) == B.VSA_ERR_UNSUPPORTED
    assert _status(f, L, B.VSA_BF16, None, k, v, None, None, 0, 0, None, ctypes.c_float(0.1), o, None,
                   None) == B.VSA_ERR_INVALID
    assert _status(f, L, B.VSA_BF16, q, k, v, _fake(8), _fake(9), 8, 3, None, ctypes.c_float(0.1), o, None,
                   None) == B.VSA_ERR_INVALID
    assert _status(f, L, B.VSA_BF16, q, k, v, None, None, 0, 0, None, ctypes.c_float(float("nan")), o, None,
                   None) == B.VSA_ERR_INVALID
    # one batch of natural Q past 2 GiB (f32, 40 heads, d = 128, 120k tokens)
    big = vsa.Layout(T=30, H=64, W=64, heads=40, head_dim=128).c()
    assert _status(f, ctypes.byref(big), B.VSA_F32, q, k, v, None, None, 0, 0, None, ctypes.c_float(0.1), o,
                   None, None) == B.VSA_ERR_UNSUPPORTED


def test_permute_pool_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=128).c()
    L = ctypes.byref(lay)
    f = "vsa_tile_permute_pool"
    src, dst, pooled = (ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(3))
    assert _status(f, L, src, dst, None, None) == B.VSA_ERR_INVALID
    assert _status(f, L, src, ctypes.c_void_p(0x20000008), pooled, None) == B.VSA_ERR_INVALID
    assert _status(f, L, src, ctypes.c_void_p(0x10001000), pooled, None) == B.VSA_ERR_INVALID   # overlap
    assert _status(f, L, src, dst, ctypes.c_void_p(0x20000100), None) == B.VSA_ERR_INVALID      # overlap
    lay12 = vsa.Layout(T=21, H=30, W=52, heads=2, head_dim=12).c()
    assert _status(f, ctypes.byref(lay12), src, dst, pooled, None) == B.VSA_ERR_UNSUPPORTED
    g = "vsa_build_mask_topk_pooled"
    qp, kp = _fake(1), _fake(2)
    assert _status(g, L, None, kp, ctypes.c_float(0.1), 32, ctypes.c_float(0.0), 0, 32, FAKE, FAKE,
                   None, FAKE, 1 << 40, None) == B.VSA_ERR_INVALID
    assert _status(g, L, ctypes.c_void_p(0x100002), kp, ctypes.c_float(0.1), 32, ctypes.c_float(0.0),
                   0, 32, FAKE, FAKE, None, FAKE, 1 << 40, None) == B.VSA_ERR_INVALID
    # routing from pooled means needs no workspace; a misaligned mean is still rejected
    assert _status(g, L, qp, ctypes.c_void_p(0x200008), ctypes.c_float(0.1), 32, ctypes.c_float(0.0),
                   0, 32, FAKE, FAKE, None, None, 0, None) == B.VSA_ERR_INVALID
    assert _status(g, L, qp, kp, ctypes.c_float(0.1), 0, ctypes.c_float(0.9), 16, 600, FAKE, FAKE,
                   None, FAKE, 1 << 40, None) == B.VSA_ERR_INVALID


def test_slice_over_2gib_rejected_before_launch():
    """One (batch, head) slice of tiled f32 Q/K/V past 2 GiB (64 x 256 x 256
    tokens, d = 128: exactly 2^31 bytes) cannot be addressed with 32-bit
    buffer offsets: UNSUPPORTED from the forward and the backward."""
    lay = vsa.Layout(T=64, H=256, W=256, heads=1, head_dim=128).c()
    L = ctypes.byref(lay)
    far = [ctypes.c_void_p((i + 1) << 33) for i in range(12)]    # 8 GiB apart: no overlaps
    q, k, v, o = far[:4]
    assert _status("vsa_block_sparse_attn_fwd", L, B.VSA_F32, q, k, v, None, None, None, None, None,
                   0, 0, None, ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_UNSUPPORTED
    assert b"2 GiB" in B.lib().vsa_last_error()
    ws = B.lib().vsa_block_sparse_attn_bwd_workspace(L)
    assert _status("vsa_block_sparse_attn_bwd", L, B.VSA_F32, q, k, v, o, far[4], far[5], None, None,
                   0, None, None, 0, ctypes.c_float(0.1), far[6], far[7], far[8], far[9], ws,
                   None) == B.VSA_ERR_UNSUPPORTED
    assert b"2 GiB" in B.lib().vsa_last_error()


def test_noalloc_backward_rejects_layouts_past_its_scratch():
    """The allocation-free backward checks the row count against its built-in
    32 MiB scratch before anything else touches the GPU (64 heads of the 768p
    Skiparse grid are 5,160,960 rows, past the 4,194,304 it holds)."""
    lay = vsa.Layout(T=21, H=48, W=80, heads=64, head_dim=128, kind="skiparse2d").c()
    L = ctypes.byref(lay)
    p = [_fake(i) for i in range(8)]
    st = _status("vsa_block_sparse_attn_bwd_noalloc", L, B.VSA_BF16, p[0], p[1], p[2], p[3], p[4],
                 p[5], None, None, 0, None, None, 0, ctypes.c_float(0.1), p[6], p[7], _fake(9), None)
    assert st == B.VSA_ERR_UNSUPPORTED
    assert b"scratch" in B.lib().vsa_last_error()
    # the shared argument checks run first: a null gradient is rejected the same way
    st = _status("vsa_block_sparse_attn_bwd_noalloc", L, B.VSA_BF16, p[0], p[1], p[2], p[3], p[4],
                 p[5], None, None, 0, None, None, 0, ctypes.c_float(0.1), None, p[7], _fake(9), None)
    assert st == B.VSA_ERR_INVALID


def test_fused_natural_calls_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=128).c()
    L = ctypes.byref(lay)
    x, c, s, p = _fake(1), _fake(2), _fake(3), _fake(4)
    f = "vsa_quant_fp8_tiles_nat"
    assert _status(f, L, None, c, s, p, 0, None) == B.VSA_ERR_INVALID
    assert _status(f, L, x, c, s, ctypes.c_void_p(0x400004), 0, None) == B.VSA_ERR_INVALID   # pooled misaligned
    assert _status(f, L, x, x, s, None, 0, None) == B.VSA_ERR_INVALID                          # overlap
    lay48 = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=48, tile=(4, 4, 4)).c()
    assert _status(f, ctypes.byref(lay48), x, c, s, None, 1, None) == B.VSA_ERR_UNSUPPORTED  # operand layout
    big = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=256, tile=(4, 8, 8)).c()
    assert _status(f, ctypes.byref(big), x, c, s, None, 0, None) == B.VSA_ERR_UNSUPPORTED    # tile too big
    g = "vsa_block_sparse_attn_fwd_fp8_nat"
    q, k, v, o = _fake(5), _fake(6), _fake(7), _fake(8)
    args = lambda dt, sc: (L, dt, q, k, v, sc, sc, sc, None, None, 0, 0, None, ctypes.c_float(0.1), o, None, None)
    assert _status(g, *args(B.VSA_BF16, s)) == B.VSA_ERR_UNSUPPORTED
    assert _status(g, *args(B.VSA_FP8_E4M3, None)) == B.VSA_ERR_INVALID
    lay64 = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=64).c()
    assert _status(g, ctypes.byref(lay64), B.VSA_FP8_E4M3, q, k, v, s, s, s, None, None, 0, 0,
                   None, ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_UNSUPPORTED


def test_work_order_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=45, W=80, heads=40, head_dim=128).c()
    L = ctypes.byref(lay)
    f = "vsa_build_work_order"
    assert _status(f, L, None, _fake(1), None) == B.VSA_ERR_INVALID
    assert _status(f, L, ctypes.c_void_p(0x400002), _fake(1), None) == B.VSA_ERR_INVALID   # misaligned
    assert _status(f, L, _fake(1), _fake(1), None) == B.VSA_ERR_INVALID                    # overlap
    big = vsa.Layout(T=64, H=128, W=128, heads=2, head_dim=128).c()                      # 16,384 tiles
    assert _status(f, ctypes.byref(big), _fake(1), _fake(2), None) == B.VSA_ERR_UNSUPPORTED
    # the attention takes an order only with per-head lists
    q, k, v, o, wo = (_fake(i) for i in range(3, 8))
    g = "vsa_block_sparse_attn_fwd"
    assert _status(g, L, B.VSA_BF16, q, k, v, None, None, None, _fake(9), _fake(10), 8, 0, wo,
                   ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_INVALID
    assert _status(g, L, B.VSA_BF16, q, k, v, None, None, None, None, None, 0, 1, wo,
                   ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_INVALID
    assert _status(g, L, B.VSA_BF16, q, k, v, None, None, None, _fake(9), _fake(10), 8, 1,
                   ctypes.c_void_p(0x400002), ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_INVALID
    assert b"work_order" in B.lib().vsa_last_error()
    n = "vsa_block_sparse_attn_fwd_nat"
    assert _status(n, L, B.VSA_BF16, q, k, v, _fake(9), _fake(10), 8, 2, wo, ctypes.c_float(0.1), o,
                   None, None) == B.VSA_ERR_INVALID
    p = "vsa_block_sparse_attn_fwd_fp8_nat"
    assert _status(p, L, B.VSA_FP8_E4M3, q, k, v, o, o, o, _fake(9), _fake(10), 8, 0, wo,
                   ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_INVALID


def test_bf16_v_operand_argument_errors_before_launch():
    lay = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=128).c()
    L = ctypes.byref(lay)
    f = "vsa_tile_permute_v"
    assert _status(f, L, None, _fake(1), None) == B.VSA_ERR_INVALID
    assert _status(f, L, ctypes.c_void_p(0x400008), _fake(1), None) == B.VSA_ERR_INVALID   # misaligned
    assert _status(f, L, _fake(1), _fake(2), None) == B.VSA_ERR_INVALID                     # overlap
    c32 = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=128, tile=(2, 4, 4)).c()
    assert _status(f, ctypes.byref(c32), _fake(1), _fake(2), None) == B.VSA_ERR_UNSUPPORTED
    wide = vsa.Layout(T=21, H=45, W=80, heads=2, head_dim=264).c()
    assert _status(f, ctypes.byref(wide), _fake(1), _fake(2), None) == B.VSA_ERR_UNSUPPORTED
    # the forwards take the layout with 64-token tiles only
    q, k, v, o = (_fake(i) for i in range(3, 7))
    g = "vsa_block_sparse_attn_fwd"
    assert _status(g, ctypes.byref(c32), B.VSA_BF16_VOP, q, k, v, None, None, None, None, None, 0, 0,
                   None, ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_UNSUPPORTED
    n = "vsa_block_sparse_attn_fwd_nat"
    assert _status(n, ctypes.byref(c32), B.VSA_BF16_VOP, q, k, v, None, None, 0, 0, None,
                   ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_UNSUPPORTED
    assert b"64-token" in B.lib().vsa_last_error()
    # fp8 natural-order output does not take it
    p = "vsa_block_sparse_attn_fwd_fp8_nat"
    s = _fake(9)
    assert _status(p, L, B.VSA_BF16_VOP, q, k, v, s, s, s, None, None, 0, 0, None,
                   ctypes.c_float(0.1), o, None, None) == B.VSA_ERR_UNSUPPORTED
