"""MX (microscaling) quantisation of bf16 tensors to E4M3 + E8M0 (oracle).

opensourcebeat.com, "Enabling up to 41 % faster pre-training: MXFP8 and
DeepEP ...", FAQ "What is MXFP8?": each block of 32 elements shares one
exponent.  The block always runs along the contraction axis of the GEMM that
consumes the copy (reading of the pages, which show only the forward pass):

* row-wise   -- blocks of 32 consecutive elements of a row (X and W for the
  forward GEMM, dY for dgrad);
* column-wise -- blocks of 32 consecutive rows of one column, restarting at
  every expert's first row (dY and X for wgrad, W for dgrad).  A group's last
  block may hold fewer than 32 rows; its amax covers the real rows only.

Steps for one block v_1..v_n (n <= 32), in order:

1. amax = max |v_i| over the block.
2. shared exponent e = floor(log2 amax) - 8, where 8 = floor(log2 448) is the
   largest E4M3 exponent (the OCP MX v1.0 rule); e = -127 when amax = 0;
   e is clamped to [-127, 127]; the scale byte is e + 127.
3. q_i = E4M3(v_i * 2^-e), rounded to nearest even and saturated at 448.
   The product is exact (power-of-two scaling of a bf16 value).
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_to_f64, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode, fp4_pack, fp4_unpack

BLOCK = 32
E4M3_EMAX = 8
E2M1_EMAX = 2          # largest exponent of an E2M1 element: 6 = 1.5 * 2^2


def mx_block_exponent(amax, emax: int = E4M3_EMAX) -> np.ndarray:
    """Shared exponent of blocks with the given amax (step 2 above; emax is the element format's
    largest exponent: 8 for E4M3, 2 for E2M1)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)               # amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    e = (ex - 1) - emax
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def _quantize_blocks(v: np.ndarray, axis: int, fp4: bool = False):
    """Quantise float64 values whose blocks run along `axis` (each block whole); E4M3 codes, or
    E2M1 codes (unpacked, one per byte) with fp4."""
    amax = np.max(np.abs(v), axis=axis, keepdims=True)
    e = mx_block_exponent(amax, E2M1_EMAX if fp4 else E4M3_EMAX)
    q = (e2m1_encode if fp4 else e4m3_encode)(np.ldexp(v, -e))
    return q, (e + 127).astype(np.uint8)


def mx_quantize_rowwise(x_bits):
    """bf16 [R, C] -> (q uint8 [R, C], s uint8 [R, C/32]); blocks along each row."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    if C % BLOCK:
        raise ValueError("C must be a multiple of 32")
    v = bf16_bits_to_f64(x_bits).reshape(R, C // BLOCK, BLOCK)
    q, s = _quantize_blocks(v, axis=2)
    return q.reshape(R, C), s.reshape(R, C // BLOCK)


def mx_colwise_ld_min(M: int, G: int) -> int:
    """Smallest admissible leading dimension of the column-wise layout.

    Group g needs 32*ceil(m_g/32) <= m_g + 31 columns, so 32*ceil((M+31G)/32)
    columns hold any split of M rows into G groups.
    """
    return 32 * (-(-(M + 31 * G) // 32))


def mx_group_columns(offs):
    """First column of each group in the column-wise layout: 32 * sum_{h<g} ceil(m_h/32)."""
    offs = np.asarray(offs, dtype=np.int64)
    nb = -(-np.diff(offs) // BLOCK)
    start = np.zeros(len(nb) + 1, dtype=np.int64)
    np.cumsum(nb, out=start[1:])
    return BLOCK * start[:-1], nb


def mx_quantize_colwise(x_bits, offs, ld: int):
    """bf16 [R, C] quantised with blocks down the rows of each group.

    ``offs=None`` means a single group of all R rows (then ld >= 32*ceil(R/32)).
    W [G*N, K] for dgrad uses it: with N a multiple of 32 no block straddles
    two experts, so one group gives the per-expert blocking.

    Returns qT uint8 [C, ld] and sT uint8 [C, ld/32].  Group g occupies
    columns [c_g, c_g + m_g) with c_g = 32 * sum_{h<g} ceil(m_h/32); every
    other byte (the <= 31 pad columns after each group and the tail) is 0x00,
    and so is every scale byte that belongs to no block.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    if offs is None:                      # one group spanning all rows
        offs = np.array([0, R], dtype=np.int64)
        need = BLOCK * (-(-R // BLOCK))
    else:
        offs = np.asarray(offs, dtype=np.int64)
        need = mx_colwise_ld_min(R, len(offs) - 1)
    if offs[0] != 0 or offs[-1] != R or np.any(np.diff(offs) < 0):
        raise ValueError("bad offsets")
    if ld % BLOCK or ld < need:
        raise ValueError("bad ld")
    qT = np.zeros((C, ld), dtype=np.uint8)
    sT = np.zeros((C, ld // BLOCK), dtype=np.uint8)
    col0, nb = mx_group_columns(offs)
    for g in range(len(offs) - 1):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        for b in range(int(nb[g])):
            a = r0 + BLOCK * b
            z = min(a + BLOCK, r1)
            v = bf16_bits_to_f64(x_bits[a:z, :])          # [n, C], block along rows
            q, s = _quantize_blocks(v, axis=0)
            c = int(col0[g]) + BLOCK * b
            qT[:, c:c + (z - a)] = q.T
            sT[:, c // BLOCK] = s[0]
    return qT, sT


def mx_dequantize(q, s) -> np.ndarray:
    """Exact value of an MX array whose 32-blocks run along the last axis."""
    q = np.asarray(q)
    s = np.asarray(s).astype(np.int64)
    if q.shape[-1] != s.shape[-1] * BLOCK:
        raise ValueError("shape mismatch")
    scale = np.ldexp(1.0, s - 127)
    return e4m3_decode(q) * np.repeat(scale, BLOCK, axis=-1)


def mx_gather_rows(x_bits, row_idx):
    """Routed rows of a token matrix: row r of the result is x[row_idx[r]].

    A dropless MoE layer computes each expert on the tokens routed to it, stored
    contiguously per expert (iitak.ru, "NVIDIA sped up training of
    mixture-of-experts models on JAX tenfold": every expert on its real token
    count in one call), so the tokens are first permuted into expert order; a
    token routed to k experts appears k times.  Indices outside [0, R_src) are
    clamped (the library's documented handling of invalid device indices).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    idx = np.clip(np.asarray(row_idx, dtype=np.int64), 0, x_bits.shape[0] - 1)
    return x_bits[idx]


def mx_quantize_dual(x_bits, offs, ld: int, row_idx=None):
    """Both MX layouts of one tensor: (q, s) row-wise and (qT, sT) column-wise.

    The input side of a layer needs X, dY and W in both directions (blocks run
    along each GEMM's contraction axis); the fused quantiser produces both from
    one read, optionally gathering routed rows first.  Definition: the row-wise
    and column-wise quantisations above of x' = x (row_idx None) or of the
    routed rows x' = mx_gather_rows(x, row_idx).
    """
    xr = np.asarray(x_bits, dtype=np.uint16) if row_idx is None else mx_gather_rows(x_bits, row_idx)
    q, s = mx_quantize_rowwise(xr)
    qT, sT = mx_quantize_colwise(xr, offs, ld)
    return q, s, qT, sT


# ------------------------------------------------------------------------------------------- MXFP4
# The same block rule with E2M1 elements (OCP MX v1.0 "MXFP4"): e = floor(log2 amax) - 2, codes
# E2M1(v * 2^-e) to nearest even, saturating at 6; two codes per byte (see codecs.fp4_pack).

def mxfp4_quantize_rowwise(x_bits):
    """bf16 [R, C] -> (q uint8 [R, C/2] packed E2M1, s uint8 [R, C/32])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    if C % BLOCK:
        raise ValueError("C must be a multiple of 32")
    v = bf16_bits_to_f64(x_bits).reshape(R, C // BLOCK, BLOCK)
    q, s = _quantize_blocks(v, axis=2, fp4=True)
    return fp4_pack(q.reshape(R, C)), s.reshape(R, C // BLOCK)


def mxfp4_quantize_colwise(x_bits, offs, ld: int):
    """Column-wise MXFP4 copy in the layout of mx_quantize_colwise, codes packed along ld:
    qT uint8 [C, ld/2], sT uint8 [C, ld/32]; pads and the tail are zero."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    if offs is None:
        offs = np.array([0, R], dtype=np.int64)
        need = BLOCK * (-(-R // BLOCK))
    else:
        offs = np.asarray(offs, dtype=np.int64)
        need = mx_colwise_ld_min(R, len(offs) - 1)
    if offs[0] != 0 or offs[-1] != R or np.any(np.diff(offs) < 0):
        raise ValueError("bad offsets")
    if ld % BLOCK or ld < need:
        raise ValueError("bad ld")
    codes = np.zeros((C, ld), dtype=np.uint8)
    sT = np.zeros((C, ld // BLOCK), dtype=np.uint8)
    col0, nb = mx_group_columns(offs)
    for g in range(len(offs) - 1):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        for b in range(int(nb[g])):
            a = r0 + BLOCK * b
            z = min(a + BLOCK, r1)
            q, s = _quantize_blocks(bf16_bits_to_f64(x_bits[a:z, :]), axis=0, fp4=True)
            c = int(col0[g]) + BLOCK * b
            codes[:, c:c + (z - a)] = q.T
            sT[:, c // BLOCK] = s[0]
    return fp4_pack(codes), sT


def mxfp4_dequantize(q, s) -> np.ndarray:
    """Exact value of a packed MXFP4 array whose 32-blocks run along the last axis."""
    v = e2m1_decode(fp4_unpack(q))
    s = np.asarray(s).astype(np.int64)
    if v.shape[-1] != s.shape[-1] * BLOCK:
        raise ValueError("shape mismatch")
    return v * np.repeat(np.ldexp(1.0, s - 127), BLOCK, axis=-1)


# ---------------------------------------------------------------- gated activation + quantisation
def mx_quantize_rowwise_values(v):
    """MX-quantise exact real values (float64 [R, C], e.g. float32 results widened) row-wise: the same
    block rule as mx_quantize_rowwise, whose input is bf16 bit patterns."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the contract")
    R, C = v.shape
    if C % BLOCK:
        raise ValueError("C must be a multiple of 32")
    q, s = _quantize_blocks(v.reshape(R, C // BLOCK, BLOCK), axis=2)
    return q.reshape(R, C), s.reshape(R, C // BLOCK)


def mx_quantize_colwise_values(v, offs, ld: int):
    """MX-quantise exact real values (float64 [R, C], e.g. float32 results widened) column-wise in the
    layout of mx_quantize_colwise: blocks of 32 rows of one column restarting at every group's first
    row, group g at columns [c_g, c_g + m_g), a short last block's amax over its real rows, pads, the
    tail and scale bytes of no block 0x00.  The same block rule as mx_quantize_colwise, whose input is
    bf16 bit patterns."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the contract")
    R, C = v.shape
    offs = np.asarray(offs, dtype=np.int64)
    if offs[0] != 0 or offs[-1] != R or np.any(np.diff(offs) < 0):
        raise ValueError("bad offsets")
    if ld % BLOCK or ld < mx_colwise_ld_min(R, len(offs) - 1):
        raise ValueError("bad ld")
    qT = np.zeros((C, ld), dtype=np.uint8)
    sT = np.zeros((C, ld // BLOCK), dtype=np.uint8)
    col0, nb = mx_group_columns(offs)
    for g in range(len(offs) - 1):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        for b in range(int(nb[g])):
            a = r0 + BLOCK * b
            z = min(a + BLOCK, r1)
            q, s = _quantize_blocks(v[a:z, :], axis=0)
            c = int(col0[g]) + BLOCK * b
            qT[:, c:c + (z - a)] = q.T
            sT[:, c // BLOCK] = s[0]
    return qT, sT


TILE = 128


def mx_colwise_tiled(qT):
    """A column-wise copy qT [C, ld] in the library's 128-byte tiled layout (a layout option of the
    library, not something the pages define; the permutation is the library's stated contract): tile t
    holds columns [128 t, 128 t + 128) of every row, row c of the tile being bytes 128 t .. 128 t + 127
    of qT's row c, so byte (c, j) lands at flat position (j // 128) * C * 128 + c * 128 + j % 128.
    Returns [ld // 128, C, 128] of the same dtype; ld % 128 == 0."""
    qT = np.asarray(qT)
    C, ld = qT.shape
    if ld % TILE:
        raise ValueError("the tiled layout needs ld % 128 == 0")
    out = np.empty((ld // TILE, C, TILE), dtype=qT.dtype)
    for t in range(ld // TILE):
        out[t] = qT[:, TILE * t:TILE * (t + 1)]
    return out


def mx_scales_tiled(s):
    """The scale bytes [rows, nb] of an MX copy (row-wise s [R, C / 32] or column-wise sT [C, ld / 32]) in
    the library's tiled layout (its stated contract, as above): tile t holds blocks [4 t, 4 t + 4) of
    every row (the scales of code tile t, one 128-element slice), so scale byte (row, b) lands at flat
    position (b // 4) * rows * 4 + row * 4 + b % 4.  Returns [nb // 4, rows, 4]; nb % 4 == 0."""
    s = np.asarray(s)
    rows, nb = s.shape
    per = TILE // 32                       # blocks (scale bytes) per 128-element slice
    if nb % per:
        raise ValueError("the tiled layout needs a multiple of 128 elements per row")
    out = np.empty((nb // per, rows, per), dtype=s.dtype)
    for t in range(nb // per):
        out[t] = s[:, per * t:per * (t + 1)]
    return out


def swiglu(gate, up):
    """Gated activation of an expert's gate+up output: silu(gate) * up, silu(z) = z / (1 + e^-z).

    Reading: the pages name no activation; SwiGLU is the gated unit of the DeepSeek-V3 and Llama-4
    expert MLPs the configurations come from.  The gate+up GEMM's output columns [0, H) are the gate
    and [H, 2H) the up projection of each expert."""
    g = np.asarray(gate, dtype=np.float64)
    with np.errstate(over="ignore"):            # e^-g overflows to inf for g < -709: silu -> -0
        return g / (1.0 + np.exp(-g)) * np.asarray(up, dtype=np.float64)
