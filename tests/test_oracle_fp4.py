"""Pins for the oracle's MXFP4 path (E2M1 elements, E8M0 per 32, two codes per byte): the codec's
closed forms and a brute-force encoder, an exhaustive bf16 sweep with an independent bit-level
derivation of the scale, the MX invariants, the column-wise layout against the row-wise quantiser of
transposed groups, and the GEMMs against np.matmul and fsum loops."""
import math

import numpy as np

from oracle import (e2m1_decode, e2m1_encode, e2m1_encode_bruteforce, fp4_pack, fp4_unpack, mx_colwise_ld_min,
                    mx_group_columns, mxfp4_dequantize, mxfp4_gemm_dgrad, mxfp4_gemm_fwd, mxfp4_gemm_wgrad,
                    mxfp4_quantize_colwise, mxfp4_quantize_rowwise)
from workloads import f32_to_bf16_bits, routing_offsets


def test_e2m1_closed_forms_and_round_trip():
    vals = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(e2m1_decode(np.arange(8))) == vals
    assert list(e2m1_decode(np.arange(8, 16))) == [-v for v in vals]
    assert np.signbit(e2m1_decode(8))
    c = np.arange(16, dtype=np.uint8)
    assert np.array_equal(e2m1_encode(e2m1_decode(c)), c)


def test_e2m1_encode_against_bruteforce():
    # every midpoint, just either side of it, beyond saturation, and random reals
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    eps = 2.0 ** -20
    y = np.concatenate([mids, mids - eps, mids + eps, [6.0, 6.5, 100.0, 1e-30, 0.0],
                        np.random.default_rng(1).uniform(-8, 8, 4000)])
    y = np.concatenate([y, -y])
    assert np.array_equal(e2m1_encode(y), e2m1_encode_bruteforce(y))
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 2.5 -> 2, 5 -> 4, 7 -> 6 (saturation)
    assert list(e2m1_decode(e2m1_encode(np.array([0.25, 0.75, 1.25, 2.5, 3.5, 5.0, 7.0])))) == \
        [0, 1, 1, 2, 4, 4, 6]


def test_pack_layout():
    c = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    assert list(fp4_pack(c)[0]) == [0x21, 0x43]
    assert np.array_equal(fp4_unpack(fp4_pack(c)), c)


def _finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def test_exhaustive_bf16_as_block_max():
    """Every finite bf16 pattern as the block maximum: the scale byte from the exponent field alone
    (E - 2 for a normal value, clamped at 0; 0 for zero and subnormals), its code from the brute-force
    encoder of the value divided by the scale."""
    p = _finite_bf16()
    x = np.zeros((len(p), 32), np.uint16)
    x[:, 0] = p
    q, s = mxfp4_quantize_rowwise(x)
    E = (p.astype(np.int64) >> 7) & 0xFF
    want_s = np.where(E == 0, 0, np.maximum(E - 2, 0))
    assert np.array_equal(s[:, 0], want_s)
    v = (p.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want_q = e2m1_encode_bruteforce(np.ldexp(v, -(want_s.astype(np.int64) - 127)))
    assert np.array_equal(fp4_unpack(q)[:, 0], want_q)
    assert not fp4_unpack(q)[:, 1:].any()


def test_shift_invariance_idempotence_exactness():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((500, 64)) * np.where(rng.random((500, 64)) < 0.02, 50.0, 1.0)
    x = f32_to_bf16_bits(v.astype(np.float32))
    q, s = mxfp4_quantize_rowwise(x)
    for j in (-7, 3, 20):
        q2, s2 = mxfp4_quantize_rowwise(f32_to_bf16_bits((v * 2.0 ** j).astype(np.float32)))
        keep = (s.astype(int) + j >= 1) & (s.astype(int) + j <= 254)
        assert np.array_equal(s2[keep], (s.astype(int) + j)[keep])
        rows = np.all(keep, axis=1)
        assert np.array_equal(q2[rows], q[rows])
    d = mxfp4_dequantize(q, s)
    q3, s3 = mxfp4_quantize_rowwise(f32_to_bf16_bits(d.astype(np.float32)))
    assert np.array_equal(fp4_unpack(q3), fp4_unpack(q))
    # blocks of E2M1 values times a power of two whose amax is 6 * 2^t quantise losslessly
    c = e2m1_decode(rng.integers(0, 16, (10, 32)))
    c[:, 0] = 6.0
    xe = f32_to_bf16_bits((c * 2.0 ** -5).astype(np.float32))
    qe, se = mxfp4_quantize_rowwise(xe)
    assert np.all(se == 127 - 5) and np.array_equal(mxfp4_dequantize(qe, se), c * 2.0 ** -5)


def test_colwise_is_rowwise_of_transposed_groups():
    rng = np.random.default_rng(3)
    sizes, C = [0, 5, 70, 1, 33, 0], 64
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    x = f32_to_bf16_bits(rng.standard_normal((M, C)).astype(np.float32))
    ld = mx_colwise_ld_min(M, G) + 32
    qT, sT = mxfp4_quantize_colwise(x, offs, ld)
    assert qT.shape == (C, ld // 2)
    col0, nb = mx_group_columns(offs)
    codes = fp4_unpack(qT)
    used = np.zeros(ld, bool)
    for g in range(G):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        if r1 == r0:
            continue
        pad = np.zeros((32 * int(nb[g]), C), np.uint16)
        pad[:r1 - r0] = x[r0:r1]
        qr, sr = mxfp4_quantize_rowwise(np.ascontiguousarray(pad.T))
        c0 = int(col0[g])
        assert np.array_equal(codes[:, c0:c0 + r1 - r0], fp4_unpack(qr)[:, :r1 - r0])
        assert np.array_equal(sT[:, c0 // 32:c0 // 32 + int(nb[g])], sr)
        used[c0:c0 + r1 - r0] = True
    assert not codes[:, ~used].any()


def test_gemms_against_matmul_and_fsum():
    rng = np.random.default_rng(4)
    sizes, N, K = [3, 0, 40], 64, 96
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    bf = lambda shape, std=1.0: f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    x, w, dy = bf((M, K)), bf((G * N, K), 0.05), bf((M, N))
    qx, sx = mxfp4_quantize_rowwise(x)
    qw, sw = mxfp4_quantize_rowwise(w)
    y, _ = mxfp4_gemm_fwd(qx, sx, qw, sw, offs, N)
    X, W = mxfp4_dequantize(qx, sx), mxfp4_dequantize(qw, sw)
    grp = np.repeat(np.arange(G), sizes)
    for r, g in enumerate(grp):
        for n in range(0, N, 7):
            assert math.isclose(y[r, n], math.fsum(X[r, k] * W[g * N + n, k] for k in range(K)),
                                rel_tol=1e-12, abs_tol=1e-300)
    # dgrad against a column-wise W, wgrad against the transposed product of the group rows
    qwT, swT = mxfp4_quantize_colwise(w, None, G * N)
    qd, sd = mxfp4_quantize_rowwise(dy)
    dx, _ = mxfp4_gemm_dgrad(qd, sd, qwT, swT, offs, N, K)
    D, WT = mxfp4_dequantize(qd, sd), mxfp4_dequantize(qwT, swT)
    for r, g in enumerate(grp):
        assert np.allclose(dx[r], D[r] @ WT[:, g * N:(g + 1) * N].T, rtol=1e-12, atol=1e-300)
    ld = mx_colwise_ld_min(M, G)
    qdT, sdT = mxfp4_quantize_colwise(dy, offs, ld)
    qxT, sxT = mxfp4_quantize_colwise(x, offs, ld)
    dw, _ = mxfp4_gemm_wgrad(qdT, sdT, qxT, sxT, offs, N, K)
    DT, XT = mxfp4_dequantize(qdT, sdT), mxfp4_dequantize(qxT, sxT)
    col0, _ = mx_group_columns(offs)
    assert not dw[1].any()
    for g in (0, 2):
        c0, m = int(col0[g]), sizes[g]
        assert np.allclose(dw[g], DT[:, c0:c0 + m] @ XT[:, c0:c0 + m].T, rtol=1e-12, atol=1e-300)
