"""The Python binding checks every tensor's dtype and shape against the
layout before it calls the C ABI (which sees only pointers). Each case below
must raise ValueError on the host: the tensors are CPU tensors, so a check
that let one through would fail later on "tensors must live in GPU memory"
instead, which the message match rejects."""
import pytest
import torch

import block_sparse_attention_token_amd as vsa

LAY = vsa.Layout(T=4, H=8, W=8, heads=2, head_dim=64)        # 4 tiles of 64 tokens
N_TOK, N_PAD, N_T = 256, 256, 4
LAY_PAD = vsa.Layout(T=3, H=8, W=8, heads=2, head_dim=64)    # 3 real, 4 padded frames
TILED = (1, 2, N_PAD, 64)
NAT = (1, N_TOK, 2, 64)


def bf(shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(shape):
    return torch.zeros(shape, dtype=torch.int32)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_layout_sizes():
    info = vsa.layout_info(LAY)
    assert (info.n_tokens, info.n_padded, info.n_tiles) == (N_TOK, N_PAD, N_T)
    info = vsa.layout_info(LAY_PAD)
    assert (info.n_tokens, info.n_padded) == (192, 256)


def test_permute_checks():
    _raises("src must have dtype", vsa.tile_permute, LAY, torch.zeros(NAT, dtype=torch.float16))
    _raises("src must have shape", vsa.tile_permute, LAY, bf((1, N_TOK + 1, 2, 64)))
    _raises("src must have shape", vsa.tile_permute, LAY, bf(NAT), inverse=True)
    _raises("out must have dtype", vsa.tile_permute, LAY, bf(NAT), out=f32(TILED))
    # natural-order out of a padded layout is smaller than the tiled tensor
    _raises("out must have shape", vsa.tile_permute, LAY_PAD, bf(TILED), inverse=True,
            out=bf(TILED))


def test_permute_pool_checks():
    _raises("src must have dtype", vsa.tile_permute_pool, LAY, f32(NAT))
    _raises("out must have shape", vsa.tile_permute_pool, LAY, bf(NAT), out=bf((1, 2, 128, 64)))
    _raises("pooled must have dtype", vsa.tile_permute_pool, LAY, bf(NAT),
            pooled=bf((1, 2, N_T, 64)))


def test_routing_and_quant_take_bf16_tiles():
    _raises("q_tiled must have dtype", vsa.build_mask_topk, LAY, f32(TILED), bf(TILED), top_k=2)
    _raises("k_tiled must have shape", vsa.build_mask_topk, LAY, bf(TILED), bf(NAT), top_k=2)
    _raises("x_tiled must have dtype", vsa.quant_fp8_tiles, LAY, f32(TILED))
    _raises("x_tiled must have shape", vsa.quant_fp8_tiles, LAY, bf((1, 2, 128, 64)))
    _raises("x_tiled must have dtype", vsa.quant_fp8_tiles_grouped, LAY, f32(TILED), (1, 1, 1))
    _raises("pooled means", vsa.build_mask_topk_pooled, LAY, bf((1, 2, N_T, 64)),
            f32((1, 2, N_T, 64)), top_k=2)


def test_forward_checks():
    q = bf(TILED)
    _raises("k must have dtype", vsa.block_sparse_attn_fwd, LAY, q, f32(TILED), q)
    _raises("v must have shape", vsa.block_sparse_attn_fwd, LAY, q, q, bf((1, 2, 128, 64)))
    # int64 lists would be read as int32 pairs
    _raises("kv_idx must have dtype", vsa.block_sparse_attn_fwd, LAY, q, q, q,
            torch.zeros((N_T, 2), dtype=torch.int64), i32((N_T,)))
    _raises("kv_cnt must have shape", vsa.block_sparse_attn_fwd, LAY, q, q, q,
            i32((N_T, 2)), i32((N_T + 1,)))
    _raises("kv_idx must be", vsa.block_sparse_attn_fwd, LAY, q, q, q, i32((2, N_T, 2)), i32((2, N_T)))
    _raises("together", vsa.block_sparse_attn_fwd, LAY, q, q, q, i32((N_T, 2)), None)
    _raises("kv_idx must have shape", vsa.block_sparse_attn_fwd, LAY, q, q, q,
            i32((1, 3, N_T, 2)), i32((1, 3, N_T)))
    _raises("per_tile_walk", vsa.block_sparse_attn_fwd, LAY, q, q, q, i32((1, 2, N_T, 2)),
            i32((1, 2, N_T)), per_tile_walk=True)
    _raises("out must have dtype", vsa.block_sparse_attn_fwd, LAY, q, q, q, out=f32(TILED))
    _raises("out must have shape", vsa.block_sparse_attn_fwd, LAY, q, q, q, out=bf(NAT[:3] + (32,)))
    _raises("lse must have shape", vsa.block_sparse_attn_fwd, LAY, q, q, q, lse=f32((1, 2, 255)))
    _raises("scales apply", vsa.block_sparse_attn_fwd, LAY, q, q, q,
            scales=(f32((1, 2, N_T)),) * 3)


def test_fp8_forward_checks():
    c = torch.zeros(TILED, dtype=torch.uint8)
    s = f32((1, 2, N_T))
    _raises("need", vsa.block_sparse_attn_fwd, LAY, c, c, c)
    _raises("k must have dtype", vsa.block_sparse_attn_fwd, LAY, c, bf(TILED), c, scales=(s, s, s))
    _raises("v_scale must have shape", vsa.block_sparse_attn_fwd, LAY, c, c, c,
            scales=(s, s, f32((1, 2, N_T + 1))))
    _raises("k_scale must have dtype", vsa.block_sparse_attn_fwd, LAY, c, c, c,
            scales=(s, bf((1, 2, N_T)), s))
    _raises("v_operand applies", vsa.block_sparse_attn_fwd, LAY, f32(TILED), f32(TILED), f32(TILED),
            v_operand=True)


def test_bf16_v_operand_checks():
    _raises("src must have dtype", vsa.tile_permute_v, LAY, f32(NAT))
    _raises("src must have shape", vsa.tile_permute_v, LAY, bf(TILED))
    _raises("out must have shape", vsa.tile_permute_v, LAY_PAD, bf((1, 192, 2, 64)), out=bf((1, 2, 192, 64)))
    _raises("v_operand applies", vsa.block_sparse_attn_fwd_nat, LAY, f32(NAT), f32(TILED), f32(TILED),
            v_operand=True)


def test_natural_forward_checks():
    q = bf(NAT)
    k = bf(TILED)
    _raises("q_nat must have shape", vsa.block_sparse_attn_fwd_nat, LAY, bf(TILED), k, k)
    _raises("k must have dtype", vsa.block_sparse_attn_fwd_nat, LAY, q, f32(TILED), k)
    # a tiled-size out for a padded layout's natural output
    _raises("out must have shape", vsa.block_sparse_attn_fwd_nat, LAY_PAD, bf((1, 192, 2, 64)), k,
            k, out=bf((1, 256, 2, 64)))
    _raises("kv_idx must have dtype", vsa.block_sparse_attn_fwd_nat, LAY, q, k, k,
            torch.zeros((N_T, 2), dtype=torch.int64), i32((N_T,)))


def test_backward_checks():
    x = bf(TILED)
    lse = f32((1, 2, N_PAD))
    _raises("dout must have dtype", vsa.block_sparse_attn_bwd, LAY, x, x, x, x, f32(TILED), lse)
    _raises("lse must have shape", vsa.block_sparse_attn_bwd, LAY, x, x, x, x, x, f32((1, 2, 128)))
    _raises("out must have shape", vsa.block_sparse_attn_bwd, LAY, x, x, x, bf(NAT[:3] + (32,)), x, lse)
    _raises("q_idx must have shape", vsa.block_sparse_attn_bwd, LAY, x, x, x, x, x, lse,
            i32((N_T, 2)), i32((N_T,)), i32((N_T, 2)), i32((N_T,)))
    _raises("q_cnt must have dtype", vsa.block_sparse_attn_bwd, LAY, x, x, x, x, x, lse,
            i32((N_T, 2)), i32((N_T,)), i32((N_T, N_T)), torch.zeros((N_T,), dtype=torch.int64))
    _raises("need the forward lists", vsa.block_sparse_attn_bwd, LAY, x, x, x, x, x, lse,
            None, None, i32((N_T, N_T)), i32((N_T,)))
    _raises("dk must have shape", vsa.block_sparse_attn_bwd, LAY, x, x, x, x, x, lse,
            grads=(bf(TILED), bf((1, 2, 128, 64)), bf(TILED)))
    _raises("kv_idx must have dtype", vsa.build_transposed_lists, LAY,
            torch.zeros((N_T, 2), dtype=torch.int64), i32((N_T,)))
