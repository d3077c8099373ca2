"""Allocation-free backward (vsa_block_sparse_attn_bwd_noalloc) against the
workspace backward (vsa_block_sparse_attn_bwd): the two run the same kernels
on the same inputs, so the gradients must be bit-identical. Two calls in a
row on one process, the second on a smaller input, so that stale row
statistics left in the shared scratch by the first call would show."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_token_amd as vsa
from tests.gpu_util import announce


def _case(lay, radius, seed):
    info = vsa.layout_info(lay)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    shape = (lay.batch, info.n_tokens, lay.heads, lay.head_dim)
    q, k, v, g = (vsa.tile_permute(lay, torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
                  for _ in range(4))
    idx, cnt = vsa.build_mask_window(lay, radius)
    out, lse = vsa.block_sparse_attn_fwd(lay, q, k, v, idx, cnt, want_lse=True)
    qi, qc = vsa.build_transposed_lists(lay, idx, cnt)
    ref = vsa.block_sparse_attn_bwd(lay, q, k, v, out, g, lse, idx, cnt, qi, qc)
    grads = tuple(torch.full_like(x, 7.0) for x in (q, k, v))       # canary-filled outputs
    got = vsa.block_sparse_attn_bwd_noalloc(lay, q, k, v, out, g, lse, idx, cnt, qi, qc, grads=grads)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    return info


@pytest.mark.gpu
def test_noalloc_backward_bit_identical_two_calls():
    # 768p Skiparse sparse layer with all 40 heads: 3,225,600 rows of the 4,194,304 the scratch holds
    big = vsa.Layout(T=21, H=48, W=80, heads=40, head_dim=128, kind="skiparse2d", stride=(2, 2))
    announce("no-alloc backward: 768p Skiparse, 40 heads")
    info = _case(big, (0, 0, 0), 11)
    assert 40 * info.n_padded * 8 <= 32 << 20
    # then a small ragged 3D-window grid with padded tiles, batch 2
    small = vsa.Layout(T=5, H=9, W=13, heads=3, head_dim=128, batch=2)
    announce("no-alloc backward: ragged 5x9x13, 3 heads, batch 2")
    _case(small, (1, 1, 1), 12)


@pytest.mark.gpu
def test_noalloc_backward_dense_fp32_after_bf16():
    # dense attention (no lists) in fp32 right after the bf16 calls above
    lay = vsa.Layout(T=4, H=8, W=8, heads=2, head_dim=64, tile=(2, 4, 4))
    announce("no-alloc backward: dense fp32 4x8x8")
    info = vsa.layout_info(lay)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    shape = (1, info.n_tokens, 2, 64)
    q, k, v, g = (vsa.tile_permute(lay, torch.randn(shape, generator=gen, device="cuda")) for _ in range(4))
    out, lse = vsa.block_sparse_attn_fwd(lay, q, k, v, want_lse=True)
    ref = vsa.block_sparse_attn_bwd(lay, q, k, v, out, g, lse)
    got = vsa.block_sparse_attn_bwd_noalloc(lay, q, k, v, out, g, lse,
                                            grads=tuple(torch.empty_like(x) for x in (q, k, v)))
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
