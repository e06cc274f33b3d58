"""Pins for the oracle's MX quantisers: hand-derived worked examples, an
exhaustive bf16 sweep through an independent bit-level derivation of the scale,
and the invariants the MX block rule implies."""
import json
import os

import numpy as np
import pytest

from oracle import (bf16_bits_to_f64, e4m3_decode, e4m3_encode_bruteforce, mx_colwise_ld_min,
                    mx_dequantize, mx_quantize_colwise, mx_quantize_rowwise, mx_group_columns)
from workloads import f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_examples.json")


def _block(bits_hex):
    b = np.zeros((1, 32), dtype=np.uint16)
    for i, h in enumerate(bits_hex):
        b[0, i] = int(h, 16)
    return b


def test_rowwise_worked_examples():
    g = json.load(open(GOLD))
    for ex in g["rowwise_blocks"]:
        q, s = mx_quantize_rowwise(_block(ex["bf16"]))
        want = np.zeros(32, dtype=np.uint8)
        for i, c in enumerate(ex["codes"]):
            want[i] = int(c, 16)
        assert s[0, 0] == int(ex["scale"], 16), ex["why"]
        assert np.array_equal(q[0], want), ex["why"]


def test_colwise_worked_example():
    ex = json.load(open(GOLD))["colwise_example"]
    offs = np.array(ex["offs"])
    assert mx_colwise_ld_min(40, 3) == ex["ld"]
    x = np.zeros((40, 32), dtype=np.float32)
    x[0:3, 0] = [1, 2, 3]
    x[3:35, 0] = 0.5
    x[35:40, 0] = [4, -4, 4, -4, 1]
    qT, sT = mx_quantize_colwise(f32_to_bf16_bits(x), offs, ex["ld"])
    want = np.zeros(ex["ld"], dtype=np.uint8)
    for k, c in ex["col0_q_nonzero"].items():
        if "-" in k:
            a, b = map(int, k.split("-"))
            want[a:b + 1] = int(c, 16)
        else:
            want[int(k)] = int(c, 16)
    assert np.array_equal(qT[0], want)
    assert list(sT[0]) == ex["col0_scales"]
    assert not qT[1:].any() and not sT[1:].any()


def _scale_exponent_from_bits(bits):
    """floor(log2 |v|) - 8 from the bf16 bit fields, clamped (independent of frexp)."""
    mag = bits & 0x7FFF
    E = mag >> 7
    m = mag & 0x7F
    if mag == 0:
        return -127
    if E == 0:
        fl = (int(m).bit_length() - 1) - 133      # subnormal: m * 2^-133
    else:
        fl = int(E) - 127
    return max(-127, min(127, fl - 8))


def test_exhaustive_bf16_as_block_max():
    """Every finite bf16 pattern p as the block maximum: scale byte and code of p."""
    bits = np.array([b for b in range(65536) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
    blocks = np.zeros((len(bits), 32), dtype=np.uint16)
    blocks[:, 0] = bits
    q, s = mx_quantize_rowwise(blocks)
    exp = np.array([_scale_exponent_from_bits(int(b)) for b in bits])
    assert np.array_equal(s[:, 0].astype(np.int64), exp + 127)
    y = bf16_bits_to_f64(bits) * np.ldexp(1.0, -exp)
    sample = np.random.default_rng(0).choice(len(bits), 6000, replace=False)
    assert np.array_equal(q[sample, 0], e4m3_encode_bruteforce(y[sample]))
    # the block max always lands in [256, 512) unless the exponent was clamped
    v = np.abs(bf16_bits_to_f64(bits))
    scaled = v * np.ldexp(1.0, -exp)
    unclamped = (v > 0) & (exp > -127)
    assert np.all((scaled[unclamped] >= 256) & (scaled[unclamped] < 512))


def test_exhaustive_bf16_as_non_max_element():
    """Every finite bf16 pattern below a fixed amax: code = brute-force E4M3 of v * 2^-e."""
    bits = np.array([b for b in range(65536) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
    v = bf16_bits_to_f64(bits)
    for amax in (1.0, 3.0, 2.0 ** -100, 2.0 ** 60):
        keep = np.abs(v) <= amax
        b = bits[keep]
        blocks = np.zeros((len(b), 32), dtype=np.uint16)
        blocks[:, 0] = b
        blocks[:, 1] = f32_to_bf16_bits(np.array([amax], dtype=np.float32))[0]
        q, s = mx_quantize_rowwise(blocks)
        e = int(np.floor(np.log2(amax))) - 8
        assert np.all(s[:, 0] == e + 127)
        y = v[keep] * 2.0 ** -e
        sample = np.random.default_rng(1).choice(len(b), 3000, replace=False)
        assert np.array_equal(q[sample, 0], e4m3_encode_bruteforce(y[sample]))


def _rand_bf16(rng, shape, std=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def test_power_of_two_exactness():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 0x7F, size=(500, 32))
    codes[:, 0] = rng.integers(0x78, 0x7F, size=500)        # one element in [256, 448]
    sign = rng.integers(0, 2, size=(500, 32)) * 0x80
    t = rng.integers(-100, 100, size=(500, 1))
    v = e4m3_decode(codes | sign) * np.ldexp(1.0, t)
    bits = f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(bits), v)            # exact in bf16
    q, s = mx_quantize_rowwise(bits)
    assert np.array_equal(s[:, 0].astype(np.int64), t[:, 0] + 127)
    assert np.array_equal(mx_dequantize(q, s), v)


def test_shift_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((400, 64)).astype(np.float32)
    q0, s0 = mx_quantize_rowwise(f32_to_bf16_bits(x))
    for j in (-40, -3, 1, 17, 60):
        xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float32)
        q1, s1 = mx_quantize_rowwise(f32_to_bf16_bits(xs))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1.astype(np.int64), s0.astype(np.int64) + j)


def test_idempotence():
    rng = np.random.default_rng(4)
    x = _rand_bf16(rng, (2000, 128))
    x[rng.random(x.shape) < 0.01] = f32_to_bf16_bits(np.array([300.0], np.float32))[0]
    q, s = mx_quantize_rowwise(x)
    d = mx_dequantize(q, s)
    bits = f32_to_bf16_bits(d.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(bits), d)
    q2, s2 = mx_quantize_rowwise(bits)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_zero_and_signed_zero_blocks():
    x = np.zeros((2, 64), dtype=np.uint16)
    x[1, :] = 0x8000
    q, s = mx_quantize_rowwise(x)
    assert not s.any()
    assert not q[0].any() and np.all(q[1] == 0x80)


def test_ld_min_for_the_workload_shapes():
    assert [mx_colwise_ld_min(M, G) for M, G in ((1024, 4), (49152, 64), (65536, 8), (32768, 16))] == \
        [1152, 51136, 65792, 33280]


def test_colwise_equals_rowwise_of_transposed_groups():
    """Column-wise quantisation of a group whose size is a multiple of 32 equals the
    row-wise quantisation of that group's transpose, placed at its start column."""
    rng = np.random.default_rng(5)
    sizes = [64, 0, 32, 96, 0]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, C = int(offs[-1]), 96
    x = _rand_bf16(rng, (M, C))
    ld = mx_colwise_ld_min(M, len(sizes))
    qT, sT = mx_quantize_colwise(x, offs, ld)
    col0, nb = mx_group_columns(offs)
    for g, m in enumerate(sizes):
        if m == 0:
            continue
        r0 = int(offs[g])
        qr, sr = mx_quantize_rowwise(np.ascontiguousarray(x[r0:r0 + m].T))
        c = int(col0[g])
        assert np.array_equal(qT[:, c:c + m], qr)
        assert np.array_equal(sT[:, c // 32:c // 32 + m // 32], sr)
    assert not qT[:, M:].any() and not sT[:, M // 32:].any()


def test_colwise_ragged_groups_short_tail_and_pads():
    rng = np.random.default_rng(6)
    sizes = [17, 0, 33, 1, 70]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, C = int(offs[-1]), 64
    x = _rand_bf16(rng, (M, C))
    ld = mx_colwise_ld_min(M, len(sizes))
    qT, sT = mx_quantize_colwise(x, offs, ld)
    col0, nb = mx_group_columns(offs)
    assert list(col0) == [0, 32, 32, 96, 128] and list(nb) == [1, 0, 2, 1, 3]
    v = bf16_bits_to_f64(x)
    used = np.zeros(ld, dtype=bool)
    for g, m in enumerate(sizes):
        r0, c0 = int(offs[g]), int(col0[g])
        used[c0:c0 + m] = True
        for b in range(int(nb[g])):
            rows = slice(r0 + 32 * b, min(r0 + 32 * b + 32, r0 + m))
            amax = np.abs(v[rows]).max(axis=0)                       # per column, real rows only
            e = np.floor(np.log2(amax)).astype(np.int64) - 8
            assert np.array_equal(sT[:, c0 // 32 + b].astype(np.int64), e + 127)
    assert not qT[:, ~used].any()
    # dequantised values are within half an E4M3 step of the input, or below it by
    # the saturation error (< 1/8: a scaled block max lies in [256, 512) and saturates at 448)
    d = mx_dequantize(qT, sT)
    for g, m in enumerate(sizes):
        r0, c0 = int(offs[g]), int(col0[g])
        if m:
            err = np.abs(d[:, c0:c0 + m] - v[r0:r0 + m].T)
            assert np.all(err <= np.abs(v[r0:r0 + m].T) * 2 ** -3 + 2.0 ** -9 * np.abs(v).max())


def test_gather_rows_by_explicit_loop():
    """The routed-row gather written out row by row on a tiny top-2 routing (each token twice),
    with an out-of-range index clamped to the last token."""
    from oracle import mx_gather_rows
    rng = np.random.default_rng(5)
    x = f32_to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32))
    idx = np.array([3, 0, 4, 1, 3, 2, 0, 9, -2], dtype=np.int32)
    want = np.zeros((len(idx), 64), dtype=np.uint16)
    for r, i in enumerate(idx):
        j = 0 if i < 0 else (4 if i > 4 else i)
        for c in range(64):
            want[r, c] = x[j, c]
    assert np.array_equal(mx_gather_rows(x, idx), want)


def test_dual_is_both_layouts_of_the_routed_rows():
    """mx_quantize_dual equals row-wise and column-wise quantisation of the routed rows, and the
    row-wise codes of a permuted tensor are the permuted codes (row-wise blocks are row-local)."""
    from oracle import mx_quantize_dual
    rng = np.random.default_rng(6)
    T, C = 40, 96
    x = f32_to_bf16_bits((rng.standard_normal((T, C)) * np.where(rng.random((T, C)) < 0.02, 100, 1))
                         .astype(np.float32))
    idx = np.concatenate([rng.permutation(T), rng.permutation(T)[:25]]).astype(np.int32)   # 65 routed rows
    offs = np.array([0, 17, 17, 50, 65], dtype=np.int64)
    ld = mx_colwise_ld_min(65, 4)
    q, s, qT, sT = mx_quantize_dual(x, offs, ld, row_idx=idx)
    qx, sx = mx_quantize_rowwise(x)
    assert np.array_equal(q, qx[idx]) and np.array_equal(s, sx[idx])
    # column-wise: the routed matrix built by an explicit loop
    xr = np.stack([x[i] for i in idx])
    qo, so = mx_quantize_colwise(xr, offs, ld)
    assert np.array_equal(qT, qo) and np.array_equal(sT, so)
    # no gather: the plain two layouts
    q2, s2, qT2, sT2 = mx_quantize_dual(x, None, 64)
    assert np.array_equal(q2, qx) and np.array_equal(s2, sx)
    qo2, so2 = mx_quantize_colwise(x, None, 64)
    assert np.array_equal(qT2, qo2) and np.array_equal(sT2, so2)


def test_swiglu_against_torch_and_closed_forms():
    """silu(g) * u against torch's CPU silu (a library routine), and its closed forms."""
    import torch
    from oracle import swiglu
    rng = np.random.default_rng(7)
    g = rng.standard_normal(5000) * 6
    u = rng.standard_normal(5000)
    want = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.allclose(swiglu(g, u), want, rtol=1e-14, atol=1e-300)
    assert swiglu(0.0, 3.0) == 0.0 and swiglu(1.0, 1.0) == 1.0 / (1.0 + np.exp(-1.0))
    assert swiglu(60.0, 2.0) == 120.0 and abs(swiglu(-60.0, 2.0) + 120.0 * np.exp(-60.0)) < 1e-36


def test_quantise_values_matches_bf16_path():
    """The value quantiser equals the bf16-pattern quantiser on bf16-representable inputs, and on
    float32 values it follows the same rule (exponent from the float32 amax)."""
    from oracle import mx_quantize_rowwise_values
    rng = np.random.default_rng(8)
    x = f32_to_bf16_bits((rng.standard_normal((64, 96)) * np.where(rng.random((64, 96)) < 0.02, 100, 1))
                         .astype(np.float32))
    q1, s1 = mx_quantize_rowwise(x)
    q2, s2 = mx_quantize_rowwise_values(bf16_bits_to_f64(x))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    v = rng.standard_normal((8, 32)).astype(np.float32).astype(np.float64)
    v[0, 0] = 3.0 * 2.0 ** 20                       # amax with exponent field 127 + 21
    q, s = mx_quantize_rowwise_values(v)
    assert s[0, 0] == 127 + 21 - 8


def test_colwise_values_matches_bf16_path_and_rowwise_rule():
    """The column-wise value quantiser: on bf16-representable inputs it equals the (separately pinned)
    bf16-pattern column-wise quantiser byte for byte, pads and tail included; on float32 values each
    group's 32-row blocks equal the row-wise value quantiser applied to the group's rows transposed and
    zero-padded to a multiple of 32 (zeros neither raise an amax nor change a code); an element whose
    float32 value is not a bf16 value is quantised from its own value (brute-force nearest code)."""
    from oracle import e4m3_encode_bruteforce, mx_group_columns, mx_quantize_colwise_values, mx_quantize_rowwise_values
    rng = np.random.default_rng(9)
    sizes, C = [0, 5, 70, 1, 32, 0, 41], 64
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    M, G = int(offs[-1]), len(sizes)
    ld = mx_colwise_ld_min(M, G) + 64
    x = f32_to_bf16_bits((rng.standard_normal((M, C)) * np.where(rng.random((M, C)) < 0.02, 100, 1)).astype(np.float32))
    q1, s1 = mx_quantize_colwise(x, offs, ld)
    q2, s2 = mx_quantize_colwise_values(bf16_bits_to_f64(x), offs, ld)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    v = (rng.standard_normal((M, C)) * np.exp2(rng.integers(-20, 20, (M, C)))).astype(np.float32).astype(np.float64)
    qT, sT = mx_quantize_colwise_values(v, offs, ld)
    col0, nb = mx_group_columns(offs)
    used = np.zeros(ld, bool)
    for g in range(G):
        m = sizes[g]
        if m == 0:
            continue
        pad = np.zeros((32 * int(nb[g]), C))
        pad[:m] = v[offs[g]:offs[g + 1]]
        qr, sr = mx_quantize_rowwise_values(pad.T)                  # [C, 32 nb]
        c0 = int(col0[g])
        assert np.array_equal(qT[:, c0:c0 + m], qr[:, :m])
        assert np.array_equal(sT[:, c0 // 32:c0 // 32 + int(nb[g])], sr)
        used[c0:c0 + m] = True
        # one element per group against the brute-force encoder of its scaled value
        k = int(rng.integers(0, C))
        e = int(sr[k, 0]) - 127
        assert qT[k, c0] == e4m3_encode_bruteforce(np.ldexp(pad[0, k], -e))[0]
    assert not qT[:, ~used].any() and not sT[:, int(np.sum(nb)):].any()


def test_colwise_tiled_is_the_stated_permutation():
    """The 128-byte tiled layout (library contract): byte (c, j) of qT [C, ld] at flat position
    (j // 128) * C * 128 + c * 128 + j % 128.  Checked element by element by that formula, as a bijection
    onto the buffer, and on a case small enough to write out."""
    from oracle import mx_colwise_tiled
    rng = np.random.default_rng(71)
    for C, ld in ((3, 128), (5, 384), (32, 256)):
        qT = rng.integers(0, 256, size=(C, ld), dtype=np.uint8)
        t = mx_colwise_tiled(qT)
        assert t.shape == (ld // 128, C, 128) and t.dtype == np.uint8
        flat = t.reshape(-1)
        pos = np.empty((C, ld), dtype=np.int64)
        for c in range(C):
            for j in range(ld):
                pos[c, j] = (j // 128) * C * 128 + c * 128 + j % 128
                assert flat[pos[c, j]] == qT[c, j]
        assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(C * ld))
    # 2 rows, 256 bytes: tile 0 = row 0 bytes 0..127 then row 1 bytes 0..127; tile 1 = bytes 128..255
    qT = np.arange(512, dtype=np.int64).reshape(2, 256)
    want = np.concatenate([np.arange(0, 128), np.arange(256, 384), np.arange(128, 256), np.arange(384, 512)])
    assert np.array_equal(mx_colwise_tiled(qT).reshape(-1), want)
    with pytest.raises(ValueError):
        mx_colwise_tiled(np.zeros((2, 96), dtype=np.uint8))


def test_scales_tiled_is_the_stated_permutation():
    """The tiled layout's scales (library contract): scale byte (row, b) of s [rows, nb] at flat position
    (b // 4) * rows * 4 + row * 4 + b % 4, the four scale bytes of 128-element slice b // 4 of the row.
    Checked element by element by that formula, as a bijection onto the buffer, against the code tiling
    of a column-wise copy (the scale of code byte (c, j) sits in the same tile t = j // 128, at row c,
    slot (j % 128) // 32), for a row-wise copy from the oracle's quantiser (the scale of element (r, k)
    at tile k // 128, row r, slot (k % 128) // 32), and on a case small enough to write out."""
    from oracle import mx_colwise_tiled, mx_scales_tiled, mx_quantize_rowwise
    rng = np.random.default_rng(72)
    for C, ld in ((3, 128), (5, 384), (32, 256)):
        sT = rng.integers(0, 256, size=(C, ld // 32), dtype=np.uint8)
        t = mx_scales_tiled(sT)
        assert t.shape == (ld // 128, C, 4) and t.dtype == np.uint8
        flat = t.reshape(-1)
        pos = np.empty((C, ld // 32), dtype=np.int64)
        for c in range(C):
            for b in range(ld // 32):
                pos[c, b] = (b // 4) * C * 4 + c * 4 + b % 4
                assert flat[pos[c, b]] == sT[c, b]
        assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(C * ld // 32))
        # code byte (c, j) and its block's scale land in the same tile and row
        qT = rng.integers(0, 256, size=(C, ld), dtype=np.uint8)
        qt = mx_colwise_tiled(qT)
        for c in range(C):
            for j in range(0, ld, 32):
                assert qt[j // 128, c, j % 128] == qT[c, j] and t[j // 128, c, (j % 128) // 32] == sT[c, j // 32]
    # a row-wise copy: element (r, k)'s scale, the exponent of its block, at tile k // 128
    x = (rng.standard_normal((5, 256)) * np.exp2(rng.integers(-6, 7, size=(5, 256)))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = mx_quantize_rowwise(bits)
    ts = mx_scales_tiled(s)
    assert ts.shape == (2, 5, 4)
    for r in range(5):
        for k in range(0, 256, 32):
            assert ts[k // 128, r, (k % 128) // 32] == s[r, k // 32]
    # 2 rows, 8 blocks: tile 0 = row 0 blocks 0..3 then row 1 blocks 0..3; tile 1 = blocks 4..7
    sT = np.arange(16, dtype=np.int64).reshape(2, 8)
    want = np.array([0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15])
    assert np.array_equal(mx_scales_tiled(sT).reshape(-1), want)
    with pytest.raises(ValueError):
        mx_scales_tiled(np.zeros((2, 3), dtype=np.uint8))
