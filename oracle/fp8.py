"""FP8 e4m3 codec and per-tile quantiser.

Follows the FPSAttention summary page, "Approach": FP8 quantisation and block
sparsity share one 3D tile granularity. The pages name neither the FP8 format
nor the rounding; readings taken:
  * format: OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
    bits, subnormals, no infinities, S.1111.111 is NaN, largest finite 448;
  * one scale per (tensor, batch, head, tile) over every channel of the
    tile's real tokens; a = absmax, stored scale = fl32(a / 448);
  * codes: inv = fl32(448 / a), y = fl32(x * inv), code = round-to-nearest-
    even of y to e4m3, saturating at +-448; the sign bit follows the fp32
    sign bit (so negative values that round to zero give 0x80);
  * a = 0 gives scale 0 and all-zero codes;
  * dequantised value = decode(code) * scale.
All quantiser arithmetic is float32 on purpose: the reading fixes the
operation sequence in fp32, which makes the codes exactly reproducible.
"""
from __future__ import annotations

import numpy as np

from .layout import Layout, token_order

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of one e4m3 code, straight from the bit-field definition."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_table() -> np.ndarray:
    """All 256 code values (float64; NaN for the two NaN codes)."""
    return np.array([e4m3_decode(c) for c in range(256)])


_POS = np.array([e4m3_decode(c) for c in range(0x7F)])   # codes 0x00..0x7E, ascending


def e4m3_encode(x) -> int:
    """Round one float32 value to the nearest e4m3 code (ties to even), saturating."""
    x = np.float32(x)
    if np.isnan(x):
        return 0x7F
    neg = bool(np.signbit(x))
    a = float(abs(x))
    if a >= E4M3_MAX:
        code = 0x7E
    else:
        hi = int(np.searchsorted(_POS, a, side="left"))     # _POS[hi] >= a
        if _POS[hi] == a:
            code = hi
        else:
            lo = hi - 1
            dlo, dhi = a - _POS[lo], _POS[hi] - a
            if dlo < dhi:
                code = lo
            elif dhi < dlo:
                code = hi
            else:                      # exact midpoint: even mantissa wins
                code = lo if (lo & 1) == 0 else hi
    return code | (0x80 if neg else 0)


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    """Vectorised form of e4m3_encode over a float32 array (same rule)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    neg = np.signbit(y)
    hi = np.searchsorted(_POS, np.minimum(a, E4M3_MAX), side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    code = np.where(_POS[hi] == a, hi, np.where(pick_hi, hi, lo))
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(y), 0x7F, code | np.where(neg, 0x80, 0))
    return code.astype(np.uint8)


def quantize_tiles(x_tiled: np.ndarray, lay: Layout):
    """Per-tile e4m3 quantisation of a tiled tensor [B, heads, N_pad, d].

    Loops over tiles; each step is vectorised over (batch, head) only.
    Returns (codes uint8 [B, heads, N_pad, d], scales float32 [B, heads, n_tiles]).
    """
    order = token_order(lay).reshape(lay.n_tiles, lay.tile_tokens)
    B = x_tiled.shape[0]
    C, d = lay.tile_tokens, lay.head_dim
    x = np.asarray(x_tiled, dtype=np.float32).reshape(B, lay.heads, lay.n_tiles, C, d)
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros((B, lay.heads, lay.n_tiles), dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    for t in range(lay.n_tiles):
        real = order[t] >= 0
        blk = x[:, :, t]                                       # [B, heads, C, d]
        amax = np.abs(blk[:, :, real, :]).max(axis=(2, 3)).astype(np.float32)
        nz = amax > 0
        safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
        inv = np.where(nz, f448 / safe, np.float32(0.0)).astype(np.float32)   # fp32 divide
        y = (blk * inv[:, :, None, None]).astype(np.float32)                  # fp32 multiply
        y[:, :, ~real, :] = 0.0
        c = e4m3_encode_array(y)
        c[~nz] = 0
        codes[:, :, t] = c
        scales[:, :, t] = np.where(nz, safe / f448, np.float32(0.0)).astype(np.float32)
    return codes.reshape(B, lay.heads, lay.n_padded, d), scales


def quantize_tiles_grouped(x_tiled: np.ndarray, lay: Layout, group):
    """e4m3 quantisation with one scale per group of tiles (3D tiles only).

    FPSAttention summary, Approach: FP8 quantisation on the same (big) tiles
    as the sparsity, e.g. (6,8,8) tiles built from (1,8,8) ones. Reading: a
    is the absmax over the real tokens of every tile in the group; scale
    and codes then follow quantize_tiles with that a, and the group's scale
    is stored for each of its tiles. Returns (codes, scales) as
    quantize_tiles.
    """
    from .layout import tile_coords
    order = token_order(lay).reshape(lay.n_tiles, lay.tile_tokens)
    B = x_tiled.shape[0]
    C, d = lay.tile_tokens, lay.head_dim
    x = np.asarray(x_tiled, dtype=np.float32).reshape(B, lay.heads, lay.n_tiles, C, d)
    gt, gh, gw = group
    key = [tuple(c // g for c, g in zip(tile_coords(lay, t), (gt, gh, gw))) for t in range(lay.n_tiles)]
    members = {}
    for t, k in enumerate(key):
        members.setdefault(k, []).append(t)
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros((B, lay.heads, lay.n_tiles), dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    for tiles in members.values():
        amax = np.zeros((B, lay.heads), dtype=np.float32)
        for t in tiles:
            real = order[t] >= 0
            if real.any():
                amax = np.maximum(amax, np.abs(x[:, :, t][:, :, real, :]).max(axis=(2, 3)))
        nz = amax > 0
        safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
        inv = np.where(nz, f448 / safe, np.float32(0.0)).astype(np.float32)   # fp32 divide
        for t in tiles:
            real = order[t] >= 0
            y = (x[:, :, t] * inv[:, :, None, None]).astype(np.float32)          # fp32 multiply
            y[:, :, ~real, :] = 0.0
            c = e4m3_encode_array(y)
            c[~nz] = 0
            codes[:, :, t] = c
            scales[:, :, t] = np.where(nz, safe / f448, np.float32(0.0)).astype(np.float32)
    return codes.reshape(B, lay.heads, lay.n_padded, d), scales


def dequantize_tiles(codes: np.ndarray, scales: np.ndarray, lay: Layout) -> np.ndarray:
    """decode(code) * scale, in float64, [B, heads, N_pad, d]."""
    table = decode_table()
    B = codes.shape[0]
    v = table[codes.astype(np.int64)].reshape(B, lay.heads, lay.n_tiles, lay.tile_tokens,
                                              lay.head_dim)
    v = v * scales.astype(np.float64)[:, :, :, None, None]
    return v.reshape(B, lay.heads, lay.n_padded, lay.head_dim)


def v_operand_order() -> np.ndarray:
    """Token of a 64-token tile held at each position p (0..63) of the fp8 P.V operand.

    Layout reading (the pages are silent; FPSAttention, "Approach", runs P.V in
    FP8): per channel, position p = 32 h + 16 A + 4 B + r holds token
    t = 32 A + 8 B + 4 h + r, with h, A in 0..1 and B, r in 0..3.
    """
    tok = np.empty(64, dtype=np.int64)
    for h in range(2):
        for a in range(2):
            for b in range(4):
                for r in range(4):
                    tok[32 * h + 16 * a + 4 * b + r] = 32 * a + 8 * b + 4 * h + r
    return tok


def v_operand_layout(codes: np.ndarray, lay: Layout) -> np.ndarray:
    """Per-tile codes stored channel-major in the P.V operand order.

    64-token tiles, d = 128: tile j of each (b, head) keeps its 64 * 128 bytes,
    byte 64 c + p holding channel c of token v_operand_order()[p].
    """
    assert lay.tile_tokens == 64 and lay.head_dim == 128
    B = codes.shape[0]
    x = np.asarray(codes).reshape(B, lay.heads, lay.n_tiles, 64, 128)
    x = np.swapaxes(x[:, :, :, v_operand_order(), :], -1, -2)     # [.., channel, position]
    return np.ascontiguousarray(x).reshape(B, lay.heads, lay.n_padded, lay.head_dim)
