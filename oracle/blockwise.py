"""Blockwise ("fine-grained") FP8 quantisation, DeepSeek-V3 style (oracle).

aifind.ru, "DeepSeek-V3: a revolutionary high-performance language model with
low training cost", section "Low-precision training: FP8 Framework" and the
caption of its figure (a): activations are scaled per 1x128 tile (one row,
128 columns), weights per 128x128 block, each tile/block with its own scale.

Readings (the page gives tile shapes only): the scale is an fp32 number
s = fl32(amax / 448) computed by IEEE float32 division (s = 1 when amax = 0);
elements are q = E4M3(fl32(v / s)) with the division again in float32, then
rounded to nearest even and saturated at 448 (because s is rounded, the amax
element can land just above 448).  A weight block's amax covers all
128 x 128 entries.

Power-of-two mode (pow2=True; the pages fix no scale format beyond fp32, and
this optional mode is the plainest power-of-two variant): the scale is the
smallest power of two s with 448 * s >= amax, at least 2^-126 (the smallest
normal fp32) and 1 for an all-zero tile.  Dividing by it is exact, no element
exceeds 448, and the fp32 scales stay exact under the GEMM's promotion
products.
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_decode, e4m3_encode

TILE = 128


def pow2_scale(amax) -> np.ndarray:
    """Smallest power of two s with 448 * s >= amax, clamped below at 2^-126; 1 where amax = 0.
    The exponent starts from a guess and is stepped until 448 * 2^e >= amax > 448 * 2^(e-1)
    (every product is exact in float64)."""
    a = np.asarray(amax, dtype=np.float64)
    nz = a > 0
    e = np.where(nz, np.frexp(np.where(nz, a, 1.0))[1] - 9, 0).astype(np.int64)
    for _ in range(4):
        e = e + (nz & (448.0 * np.ldexp(1.0, e) < a))
        e = e - (nz & (448.0 * np.ldexp(1.0, e - 1) >= a))
    assert np.all(~nz | ((448.0 * np.ldexp(1.0, e) >= a) & (448.0 * np.ldexp(1.0, e - 1) < a)))
    e = np.maximum(e, -126)
    return np.where(nz, np.ldexp(1.0, e), 1.0).astype(np.float32)


def _scale_and_quantize(v32: np.ndarray, amax32: np.ndarray, pow2: bool = False):
    """v32, amax32 float32 (amax broadcastable); returns (q, s float32)."""
    if pow2:
        s = pow2_scale(amax32)
    else:
        s = (amax32 / np.float32(448.0)).astype(np.float32)      # IEEE fp32 division
        s = np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)
    y = (v32 / s).astype(np.float32)                              # IEEE fp32 division
    return e4m3_encode(y.astype(np.float64)), s


def bw_quantize_act_1x128(x_bits, pow2: bool = False):
    """bf16 [R, C] -> (q uint8 [R, C], s float32 [R, C/128]), one scale per 1x128 tile."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    if C % TILE:
        raise ValueError("C must be a multiple of 128")
    v = (x_bits.astype(np.uint32) << 16).view(np.float32).reshape(R, C // TILE, TILE)
    amax = np.max(np.abs(v), axis=2, keepdims=True)
    q, s = _scale_and_quantize(v, amax, pow2)
    return q.reshape(R, C), s.reshape(R, C // TILE)


def bw_quantize_weight_128x128(w_bits, pow2: bool = False):
    """bf16 [R, C] (R = G*N) -> (q uint8 [R, C], s float32 [R/128, C/128])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    R, C = w_bits.shape
    if R % TILE or C % TILE:
        raise ValueError("R and C must be multiples of 128")
    v = (w_bits.astype(np.uint32) << 16).view(np.float32).reshape(R // TILE, TILE, C // TILE, TILE)
    amax = np.max(np.abs(v), axis=(1, 3), keepdims=True)
    q, s = _scale_and_quantize(v, amax, pow2)
    return q.reshape(R, C), s.reshape(R // TILE, C // TILE)


def bw_dequantize_act(q, s) -> np.ndarray:
    q = np.asarray(q)
    return e4m3_decode(q) * np.repeat(np.asarray(s, dtype=np.float64), TILE, axis=-1)


def bw_dequantize_weight(q, s) -> np.ndarray:
    q = np.asarray(q)
    s = np.asarray(s, dtype=np.float64)
    return e4m3_decode(q) * np.repeat(np.repeat(s, TILE, axis=0), TILE, axis=1)


def bw_colwise_ld_min(M: int, G: int) -> int:
    """Smallest leading dimension of the column-wise blockwise layout: group g needs
    128*ceil(m_g/128) <= m_g + 127 columns, so 128*ceil((M + 127 G)/128) hold any split."""
    return TILE * (-(-(M + (TILE - 1) * G) // TILE))


def bw_group_columns(offs):
    """First column of each group in the column-wise blockwise layout and its block count:
    c_g = 128 * sum_{h<g} ceil(m_h/128)."""
    offs = np.asarray(offs, dtype=np.int64)
    nb = -(-np.diff(offs) // TILE)
    start = np.zeros(len(nb) + 1, dtype=np.int64)
    np.cumsum(nb, out=start[1:])
    return TILE * start[:-1], nb


def bw_quantize_colwise_128(x_bits, offs, ld: int, pow2: bool = False):
    """bf16 [R, C] quantised in 128-row blocks of one column, restarting at every group's first
    row -- the weight-gradient operands of the blockwise recipe, whose contraction runs over the
    tokens of one expert (reading: the page shows only the forward pass; the backward pass quantises
    along its own contraction axis, like the MX copies).

    Returns qT uint8 [C, ld] and sT float32 [C, ld/128].  Group g occupies columns
    [c_g, c_g + m_g) (see bw_group_columns); a group's last block may hold fewer than 128 rows and
    its amax covers the real rows only.  Pad and tail bytes are 0x00; scale slots of no block are 0.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    offs = np.asarray(offs, dtype=np.int64)
    if offs[0] != 0 or offs[-1] != R or np.any(np.diff(offs) < 0):
        raise ValueError("bad offsets")
    if ld % TILE or ld < bw_colwise_ld_min(R, len(offs) - 1):
        raise ValueError("bad ld")
    qT = np.zeros((C, ld), dtype=np.uint8)
    sT = np.zeros((C, ld // TILE), dtype=np.float32)
    col0, nb = bw_group_columns(offs)
    for g in range(len(offs) - 1):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        for b in range(int(nb[g])):
            a = r0 + TILE * b
            z = min(a + TILE, r1)
            v = (x_bits[a:z].astype(np.uint32) << 16).view(np.float32)     # [n, C]
            amax = np.max(np.abs(v), axis=0, keepdims=True)
            q, sc = _scale_and_quantize(v, amax, pow2)
            c = int(col0[g]) + TILE * b
            qT[:, c:c + (z - a)] = q.T
            sT[:, c // TILE] = sc[0]
    return qT, sT
