"""Pins for the oracle's power-of-two blockwise mode (the optional variant of the 1x128 / 128x128
blockwise recipe in which each tile's fp32 scale is the smallest power of two s with 448 s >= amax,
at least 2^-126, and 1 for an all-zero tile).

The scale is checked against a hand-derived table and against a brute-force search over every
exponent for every bf16 magnitude; the codes against the MX quantiser (an independently written
function) where both must agree, against exact representability, and through the column-wise
quantiser's relation to the activation quantiser of transposed groups."""
from fractions import Fraction

import numpy as np

from oracle import (bw_dequantize_act, bw_group_columns, bw_quantize_act_1x128, bw_quantize_colwise_128,
                    bw_quantize_weight_128x128, bw_colwise_ld_min, e4m3_decode, mx_quantize_rowwise, pow2_scale)
from workloads import f32_to_bf16_bits, routing_offsets


def _bf(rng, shape, std=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _vals(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_scale_hand_derived():
    # amax -> smallest power of two s with 448 s >= amax (448 = 1.75 * 2^8)
    table = [
        (448.0, 1.0),               # 448 * 2^0 = 448 >= 448, 448 * 2^-1 = 224 < 448
        (449.0, 2.0),               # just above 448 needs the next binade
        (1.0, 2.0 ** -8),           # 448 * 2^-8 = 1.75 >= 1 > 0.875
        (1.75, 2.0 ** -8),          # the boundary itself stays in the lower exponent
        (1.7578125, 2.0 ** -7),     # 1.75 + 2^-7 (bf16 mantissa 97 of 128) moves up
        (0.875, 2.0 ** -9),         # 448 * 2^-9 = 0.875 exactly
        (896.0, 2.0),               # 448 * 2 = 896 exactly
        (2.0 ** -140, 2.0 ** -126),  # below the smallest normal fp32: clamped
        (0.0, 1.0),                 # all-zero tile
    ]
    a = np.array([t[0] for t in table], np.float32)
    want = np.array([t[1] for t in table], np.float32)
    assert np.array_equal(pow2_scale(a), want)


def test_scale_bruteforce_every_bf16_magnitude():
    mags = np.arange(1, 0x7F80, dtype=np.uint32)             # every finite non-zero bf16 magnitude
    amax = (mags << 16).view(np.float32)
    got = pow2_scale(amax).astype(np.float64)
    # brute force: the smallest e in [-126, 127] with 448 * 2^e >= amax, in exact rationals, on a
    # sample spread over the whole range (all of them would take minutes with Fractions)
    idx = np.unique(np.concatenate([np.arange(0, len(mags), 97), np.arange(len(mags) - 300, len(mags))]))
    for i in idx:
        x = Fraction(float(amax[i]))
        e = next(e for e in range(-126, 128) if 448 * Fraction(2) ** e >= x)
        assert got[i] == float(Fraction(2) ** e), (hex(mags[i]), got[i], e)
    # and on all of them: a power of two, large enough, and minimal unless clamped
    m, ex = np.frexp(got)
    assert np.all(m == 0.5)
    assert np.all(448.0 * got >= amax)
    assert np.all((448.0 * got / 2 < amax) | (got == 2.0 ** -126))


def test_codes_never_saturate_and_are_exact_when_representable():
    rng = np.random.default_rng(30)
    x = _bf(rng, (64, 512), 3.0)
    x[5, 7] = f32_to_bf16_bits(np.array([7.0e4], np.float32))[0]       # an outlier
    q, s = bw_quantize_act_1x128(x, pow2=True)
    d = e4m3_decode(q)
    assert np.abs(d).max() <= 448.0
    v = _vals(x).astype(np.float64)
    sr = np.repeat(s.astype(np.float64), 128, axis=1)
    # every code is the nearest E4M3 value of v / s: within half an E4M3 step of it
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(v / sr), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(d - v / sr) <= step / 2)
    # values that are E4M3 numbers times a power-of-two scale come back unchanged
    c = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))                 # 0 .. 448
    t = np.zeros((1, 128), np.float32)
    t[0, :127] = c * 2.0 ** -20
    t[0, 127] = -448 * 2.0 ** -20
    qt, st = bw_quantize_act_1x128(f32_to_bf16_bits(t), pow2=True)
    assert st[0, 0] == 2.0 ** -20
    assert np.array_equal(bw_dequantize_act(qt, st), t.astype(np.float64))


def test_agrees_with_mx_when_mx_does_not_saturate():
    """A 1x128 tile whose four 32-blocks share one amax with leading significand <= 1.75: the MX rule
    (2^(floor(log2 amax) - 8)) and the power-of-two rule give the same scale, so the codes agree; above
    1.75 the power-of-two scale is twice the MX one."""
    rng = np.random.default_rng(31)
    rows = []
    amaxes = [1.5 * 2.0 ** -30, 1.75, 1.0, 1.7578125 * 2.0 ** 10, 1.9921875]
    for am in amaxes:
        v = np.clip(rng.standard_normal(128).astype(np.float32) * am / 3, -am * 0.99, am * 0.99)
        v[::32] = am
        rows.append(v)
    x = f32_to_bf16_bits(np.array(rows, np.float32))
    q, s = bw_quantize_act_1x128(x, pow2=True)
    mq, ms = mx_quantize_rowwise(x)
    for r, am in enumerate(amaxes):
        mx_scale = 2.0 ** (int(ms[r, 0]) - 127)
        assert np.all(ms[r] == ms[r, 0])
        if np.frexp(am)[0] * 2 <= 1.75:
            assert s[r, 0] == mx_scale and np.array_equal(q[r], mq[r])
        else:
            assert s[r, 0] == 2 * mx_scale


def test_weight_blocks_and_colwise_follow_the_same_rule():
    rng = np.random.default_rng(32)
    w = _bf(rng, (256, 384), 0.02)
    qw, sw = bw_quantize_weight_128x128(w, pow2=True)
    v = _vals(w)
    for i in range(2):
        for j in range(3):
            blk = v[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            assert sw[i, j] == pow2_scale(np.abs(blk).max())
    # column-wise (128-token blocks restarting per expert) equals the activation quantiser applied to
    # each expert's transposed 128-row blocks
    sizes = [130, 0, 5, 128]
    offs = routing_offsets(sizes)
    M = int(offs[-1])
    x = _bf(rng, (M, 256))
    ld = bw_colwise_ld_min(M, len(sizes))
    qT, sT = bw_quantize_colwise_128(x, offs, ld, pow2=True)
    col0, nb = bw_group_columns(offs)
    for g in range(len(sizes)):
        for b in range(int(nb[g])):
            a, z = int(offs[g]) + 128 * b, min(int(offs[g]) + 128 * (b + 1), int(offs[g + 1]))
            blk = np.zeros((256, 128), np.uint16)
            blk[:, :z - a] = x[a:z].T
            qa, sa = bw_quantize_act_1x128(blk, pow2=True)
            c = int(col0[g]) + 128 * b
            assert np.array_equal(qT[:, c:c + z - a], qa[:, :z - a])
            assert np.array_equal(sT[:, c // 128], sa[:, 0])
