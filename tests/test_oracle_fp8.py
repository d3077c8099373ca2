"""Pins for the oracle's e4m3 codec and per-tile quantiser."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8 as F
from oracle import layout as L
from oracle.layout import Layout
from tests.conftest import read_golden


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("line", read_golden("e4m3_codes.txt"))
def test_golden_codes(line):
    code_s, val_s = line.split()
    code = int(code_s, 16)
    v = F.e4m3_decode(code)
    if val_s == "nan":
        assert math.isnan(v)
    else:
        assert v == float(val_s) and math.copysign(1.0, v) == math.copysign(1.0, float(val_s))


def test_decode_matches_torch_for_all_codes():
    ours = F.decode_table()
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_encode_decode_roundtrip_all_finite_codes():
    for c in range(256):
        v = F.e4m3_decode(c)
        if math.isnan(v):
            continue
        assert F.e4m3_encode(np.float32(v)) == c


def test_midpoints_round_to_even():
    pos = [F.e4m3_decode(c) for c in range(0x7F)]
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)        # exact in fp32
        assert float(mid) == (pos[c] + pos[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode(mid) == want
        assert F.e4m3_encode(-mid) == want | 0x80
        assert F.e4m3_encode(np.nextafter(mid, np.float32(0))) == c
        assert F.e4m3_encode(np.nextafter(mid, np.float32(1000))) == c + 1


def test_saturation_and_nan():
    assert F.e4m3_encode(np.float32(448.0)) == 0x7E
    assert F.e4m3_encode(np.float32(448.01)) == 0x7E
    assert F.e4m3_encode(np.float32(1e30)) == 0x7E
    assert F.e4m3_encode(np.float32(-600.0)) == 0xFE
    assert F.e4m3_encode(np.float32("nan")) == 0x7F
    assert F.e4m3_encode(np.float32(-1e-30)) == 0x80


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 10,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_encode_array(x)
    assert np.array_equal(ours, ref)
    # scalar and vector forms agree
    for v in x[:500]:
        assert F.e4m3_encode(v) == F.e4m3_encode_array(np.array([v]))[0]


def test_quantize_tiles_properties():
    lay = Layout(T=3, H=5, W=6, heads=2, head_dim=16, tile=(2, 4, 4))
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((1, lay.n_tokens, 2, 16)) * 3).astype(np.float32)
    xt = L.permute(x, lay)
    xt[0, 1, :lay.tile_tokens] = 0.0                    # one all-zero tile
    codes, scales = F.quantize_tiles(xt, lay)
    order = L.token_order(lay).reshape(lay.n_tiles, lay.tile_tokens)
    C = lay.tile_tokens
    for h in range(2):
        for t in range(lay.n_tiles):
            blk = xt[0, h, t * C:(t + 1) * C]
            real = order[t] >= 0
            a = np.float32(np.abs(blk[real]).max())
            cb = codes[0, h, t * C:(t + 1) * C]
            if a == 0:
                assert scales[0, h, t] == 0 and np.all(cb == 0)
                continue
            assert scales[0, h, t] == np.float32(a / np.float32(448.0))
            assert np.max(cb & 0x7F) == 0x7E                # absmax maps to 448
            assert np.all(cb[~real] == 0)
    deq = F.dequantize_tiles(codes, scales, lay)
    err = np.abs(deq - xt.astype(np.float64))
    # 3 mantissa bits: relative error <= 2^-4 above the subnormal range, plus
    # an absolute floor of half the smallest subnormal step times the scale
    bound = np.abs(xt) * 2.0 ** -4 * (1 + 1e-6) + \
        scales.repeat(C, axis=2)[..., None] * 2.0 ** -10 * (1 + 1e-6)
    assert np.all(err <= bound)


def _golden_v_order():
    return [tuple(int(x) for x in line.split(":")) for line in read_golden("fp8_v_operand_order.txt")]


def test_v_operand_order_golden_and_inverse():
    tok = F.v_operand_order()
    assert sorted(tok.tolist()) == list(range(64))                  # a permutation
    for p, t in _golden_v_order():
        assert tok[p] == t, (p, t)
    # the inverse written the other way round: token t sits at
    # p = 32 ((t div 4) mod 2) + 16 (t div 32) + 4 ((t div 8) mod 4) + t mod 4
    for t in range(64):
        p = 32 * ((t // 4) % 2) + 16 * (t // 32) + 4 * ((t // 8) % 4) + t % 4
        assert tok[p] == t


def test_v_operand_layout_is_a_per_tile_transpose():
    lay = Layout(T=4, H=8, W=8, heads=2, head_dim=128, tile=(4, 4, 4))
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 256, (1, 2, lay.n_padded, 128), dtype=np.uint8)
    out = F.v_operand_layout(codes, lay)
    assert out.shape == codes.shape and out.dtype == codes.dtype
    tok = F.v_operand_order()
    for h in range(2):
        for j in range(lay.n_tiles):
            tile_in = codes[0, h, 64 * j:64 * (j + 1)]               # [token, channel]
            tile_out = out[0, h, 64 * j:64 * (j + 1)].reshape(-1)    # bytes 64 c + p
            for c in (0, 1, 77, 127):
                for p in (0, 5, 31, 32, 50, 63):
                    assert tile_out[64 * c + p] == tile_in[tok[p], c]
    # same multiset of bytes per tile: nothing lost or duplicated
    a = np.sort(codes.reshape(1, 2, lay.n_tiles, -1), axis=-1)
    b = np.sort(out.reshape(1, 2, lay.n_tiles, -1), axis=-1)
    assert np.array_equal(a, b)


def _golden_quant_cases():
    rows = []
    for line in read_golden("quant_cases.txt"):
        a_s, x_s, c_s = line.split()
        rows.append((float(a_s), float(x_s), int(c_s, 16)))
    return rows


def _one_tile(a, x):
    """A one-tile layout (one token, d = 8) whose tile holds a (its absmax) and x."""
    lay = Layout(T=1, H=1, W=1, heads=1, head_dim=8, tile=(1, 1, 1))
    t = np.zeros((1, 1, lay.n_padded, 8), dtype=np.float32)
    t[0, 0, 0, 0] = a
    t[0, 0, 0, 1] = x
    return lay, t


@pytest.mark.parametrize("a,x,code", _golden_quant_cases())
def test_quantiser_operation_order_golden(a, x, code):
    """Hand-derived codes at exact rounding midpoints (tests/golden/quant_cases.txt):
    the codes follow inv = fl32(448 / a), y = fl32(x * inv), RNE."""
    assert np.float32(x) == x and (np.float32(x).view(np.uint32) & 0xFFFF) == 0   # x is a bf16 value
    lay, t = _one_tile(a, x)
    codes, scales = F.quantize_tiles(t, lay)
    assert int(codes[0, 0, 0, 1]) == code
    assert int(codes[0, 0, 0, 0]) == 0x7E                  # the absmax itself maps to 448
    assert scales[0, 0, 0] == np.float32(np.float32(a) / np.float32(448.0))


def test_golden_quant_cases_separate_the_operation_orders():
    """The golden rows reject the two nearby readings: dividing by fl32(a / 448),
    and forming x * 448 / a in float64 before the e4m3 rounding. (Each row's
    float64 product is the exact midpoint, so float64 rounds to the even code.)"""
    by_div = by_f64 = 0
    for a, x, code in _golden_quant_cases():
        s = np.float32(np.float32(a) / np.float32(448.0))
        y_div = np.float32(np.float32(x) / s)
        by_div += F.e4m3_encode(y_div) != code
        exact = x * 448.0 / a                       # exact in float64 for these rows
        assert exact == np.float32(exact)
        by_f64 += F.e4m3_encode(np.float32(exact)) != code
    assert by_div >= 1 and by_f64 >= 1
