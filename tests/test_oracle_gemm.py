"""Pins for the oracle's grouped GEMMs: dense masked GEMM, G = 1 reduces to
np.matmul, empty groups, brute-force loops (exactly summed with math.fsum) on
tiny shapes, integer-exact inputs, and the blockwise recipe against MX where the
two coincide."""
import math

import numpy as np

from oracle import (bw_dequantize_act, bw_dequantize_weight, bw_gemm_dgrad, bw_gemm_fwd,
                    bw_quantize_act_1x128, bw_quantize_weight_128x128, check_gemm, e4m3_decode,
                    mx_colwise_ld_min, mx_dequantize, mx_gemm_dgrad, mx_gemm_fwd, mx_gemm_wgrad,
                    mx_group_columns, mx_quantize_colwise, mx_quantize_rowwise, gemm_tolerance)
from workloads import f32_to_bf16_bits, routing_offsets


def _bf(rng, shape, std=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _layer(rng, sizes, N, K):
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    return offs, _bf(rng, (M, K)), _bf(rng, (G * N, K), 0.05), _bf(rng, (M, N))


def test_fwd_equals_dense_masked_gemm():
    rng = np.random.default_rng(10)
    sizes, N, K = [5, 0, 40, 1, 19], 64, 96
    offs, x, w, _ = _layer(rng, sizes, N, K)
    qx, sx = mx_quantize_rowwise(x)
    qw, sw = mx_quantize_rowwise(w)
    y, bound = mx_gemm_fwd(qx, sx, qw, sw, offs, N)
    A, B = mx_dequantize(qx, sx), mx_dequantize(qw, sw)
    dense = A @ B.T                                     # [M, G*N]
    grp = np.repeat(np.arange(len(sizes)), sizes)
    want = np.stack([dense[r, g * N:(g + 1) * N] for r, g in enumerate(grp)])
    assert np.allclose(y, want, rtol=1e-13, atol=0)
    assert np.allclose(bound, np.stack([(np.abs(A) @ np.abs(B).T)[r, g * N:(g + 1) * N]
                                        for r, g in enumerate(grp)]), rtol=1e-13)


def test_single_group_is_plain_matmul():
    rng = np.random.default_rng(11)
    offs, x, w, dy = _layer(rng, [77], 32, 64)
    qx, sx = mx_quantize_rowwise(x)
    qw, sw = mx_quantize_rowwise(w)
    y, _ = mx_gemm_fwd(qx, sx, qw, sw, offs, 32)
    assert np.array_equal(y, np.matmul(mx_dequantize(qx, sx), mx_dequantize(qw, sw).T))


def _fsum_dot(a, b):
    return math.fsum(float(p) * float(q) for p, q in zip(a, b))


def test_bruteforce_all_three_gemms():
    rng = np.random.default_rng(12)
    sizes, N, K = [0, 1, 17, 33], 32, 64
    offs, x, w, dy = _layer(rng, sizes, N, K)
    G, M = len(sizes), int(offs[-1])
    qx, sx = mx_quantize_rowwise(x)
    qw, sw = mx_quantize_rowwise(w)
    qdy, sdy = mx_quantize_rowwise(dy)
    qwT, swT = mx_quantize_colwise(w, None, G * N)
    wT_offs = np.arange(G + 1, dtype=np.int32) * N
    qwT2, swT2 = mx_quantize_colwise(w, wT_offs, mx_colwise_ld_min(G * N, G))
    assert np.array_equal(qwT2[:, :G * N], qwT) and not qwT2[:, G * N:].any()
    ld = mx_colwise_ld_min(M, G)
    qdyT, sdyT = mx_quantize_colwise(dy, offs, ld)
    qxT, sxT = mx_quantize_colwise(x, offs, ld)
    X, W, DY = mx_dequantize(qx, sx), mx_dequantize(qw, sw), mx_dequantize(qdy, sdy)
    WT, DYT, XT = mx_dequantize(qwT, swT), mx_dequantize(qdyT, sdyT), mx_dequantize(qxT, sxT)
    y, _ = mx_gemm_fwd(qx, sx, qw, sw, offs, N)
    dx, _ = mx_gemm_dgrad(qdy, sdy, qwT, swT, offs, N, K)
    dw, _ = mx_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, N, K)
    col0, _ = mx_group_columns(offs)
    for g in range(G):
        for r in range(offs[g], offs[g + 1]):
            for n in range(N):
                assert math.isclose(y[r, n], _fsum_dot(X[r], W[g * N + n]), rel_tol=1e-12, abs_tol=1e-300)
            for k in range(K):
                assert math.isclose(dx[r, k], _fsum_dot(DY[r], WT[k, g * N:(g + 1) * N]), rel_tol=1e-12,
                                    abs_tol=1e-300)
        m, c = int(offs[g + 1] - offs[g]), int(col0[g])
        for n in range(0, N, 7):
            for k in range(0, K, 5):
                want = _fsum_dot(DYT[n, c:c + m], XT[k, c:c + m])
                assert math.isclose(dw[g, n, k], want, rel_tol=1e-12, abs_tol=1e-300)
    assert not dw[0].any()                       # empty group -> zero weight gradient


def test_wgrad_equals_transposed_product_of_group_rows():
    """dW_g = dY_g^T X_g when both column-wise copies are dequantised back to rows."""
    rng = np.random.default_rng(13)
    sizes, N, K = [40, 0, 64, 9], 32, 64
    offs, x, _, dy = _layer(rng, sizes, N, K)
    M, G = int(offs[-1]), len(sizes)
    ld = mx_colwise_ld_min(M, G)
    qdyT, sdyT = mx_quantize_colwise(dy, offs, ld)
    qxT, sxT = mx_quantize_colwise(x, offs, ld)
    dw, _ = mx_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, N, K)
    col0, _ = mx_group_columns(offs)
    DYT, XT = mx_dequantize(qdyT, sdyT), mx_dequantize(qxT, sxT)
    for g in range(G):
        m, c = sizes[g], int(col0[g])
        dYg, Xg = DYT[:, c:c + m].T, XT[:, c:c + m].T           # back to [m, N], [m, K]
        assert np.allclose(dw[g], dYg.T @ Xg, rtol=1e-13, atol=0)


def test_integer_exact_inputs():
    """Small-integer operands: every product and partial sum is an exact small integer."""
    rng = np.random.default_rng(14)
    sizes, N, K = [3, 0, 12], 32, 64
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    xi = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    wi = rng.integers(-4, 5, size=(G * N, K)).astype(np.float32)
    xi[:, ::32] = 8.0                         # every block has amax 8 -> e = -5, still exact
    wi[:, ::32] = 8.0
    qx, sx = mx_quantize_rowwise(f32_to_bf16_bits(xi))
    qw, sw = mx_quantize_rowwise(f32_to_bf16_bits(wi))
    assert np.array_equal(mx_dequantize(qx, sx), xi)
    y, _ = mx_gemm_fwd(qx, sx, qw, sw, offs, N)
    grp = np.repeat(np.arange(G), sizes)
    want = np.stack([xi[r].astype(np.int64) @ wi[g * N:(g + 1) * N].astype(np.int64).T
                     for r, g in enumerate(grp)])
    assert np.array_equal(y, want.astype(np.float64))


def test_unit_scales_reduce_to_plain_fp8_gemm():
    rng = np.random.default_rng(15)
    M, N, K = 20, 32, 64
    qx = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) * 0x80).astype(np.uint8)
    qw = rng.integers(0, 0x7F, size=(N, K)).astype(np.uint8)
    s1 = np.full((M, K // 32), 127, np.uint8)
    s2 = np.full((N, K // 32), 127, np.uint8)
    y, _ = mx_gemm_fwd(qx, s1, qw, s2, np.array([0, M], np.int32), N)
    assert np.array_equal(y, e4m3_decode(qx) @ e4m3_decode(qw).T)


def test_blockwise_quantisers_definition():
    rng = np.random.default_rng(16)
    x = _bf(rng, (6, 256))
    q, s = bw_quantize_act_1x128(x)
    v = (x.astype(np.uint32) << 16).view(np.float32)
    for r in range(6):
        for t in range(2):
            amax = np.float32(np.abs(v[r, 128 * t:128 * (t + 1)]).max())
            assert s[r, t] == np.float32(amax / np.float32(448))
    # a zero tile gets scale 1 and zero codes
    z = np.zeros((1, 128), np.uint16)
    qz, sz = bw_quantize_act_1x128(z)
    assert sz[0, 0] == 1.0 and not qz.any()
    w = _bf(rng, (256, 256), 0.02)
    qw, sw = bw_quantize_weight_128x128(w)
    vw = (w.astype(np.uint32) << 16).view(np.float32)
    assert sw.shape == (2, 2)
    assert sw[1, 0] == np.float32(np.float32(np.abs(vw[128:, :128]).max()) / np.float32(448))
    # dequantised values are within E4M3 precision of the input
    d = bw_dequantize_weight(qw, sw)
    assert np.all(np.abs(d - vw) <= np.abs(vw) * 2 ** -4 + 2.0 ** -9 * np.repeat(np.repeat(sw, 128, 0), 128, 1))


def test_blockwise_equals_mx_for_power_of_two_scales():
    """If every 32-block and every 128-tile has amax = 448 * 2^t (same t), both
    recipes pick the scale 2^t and quantise identically; so do their GEMMs."""
    rng = np.random.default_rng(17)
    sizes, N, K = [0, 130, 5], 128, 256
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    def make(rows, t):
        v = (rng.standard_normal((rows, K)) * 40).astype(np.float32)
        v = np.clip(v, -440, 440)
        v[:, ::32] = 448.0
        return f32_to_bf16_bits((v.astype(np.float64) * 2.0 ** t).astype(np.float32))
    x, w = make(M, -3), make(G * N, -9)
    qa, sa = bw_quantize_act_1x128(x)
    qw, sw = bw_quantize_weight_128x128(w)
    mqa, msa = mx_quantize_rowwise(x)
    mqw, msw = mx_quantize_rowwise(w)
    assert np.array_equal(qa, mqa) and np.array_equal(qw, mqw)
    assert np.all(sa == 2.0 ** -3) and np.all(sw == 2.0 ** -9)
    yb, bb = bw_gemm_fwd(qa, sa, qw, sw, offs, N)
    ym, bm = mx_gemm_fwd(mqa, msa, mqw, msw, offs, N)
    assert np.allclose(yb, ym, rtol=1e-12, atol=0) and np.allclose(bb, bm, rtol=1e-12)
    # dgrad: dY quantised 1x128 along N against the transposed weight blocks
    dy = make(M, 0)[:, :N].copy()
    qd, sd = bw_quantize_act_1x128(dy)
    dxb, _ = bw_gemm_dgrad(qd, sd, qw, sw, offs, N, K)
    D, Wd = bw_dequantize_act(qd, sd), bw_dequantize_weight(qw, sw)
    grp = np.repeat(np.arange(G), sizes)
    want = np.stack([D[r] @ Wd[g * N:(g + 1) * N] for r, g in enumerate(grp)]) if M else np.zeros((0, K))
    assert np.allclose(dxb, want, rtol=1e-12, atol=1e-300)


def test_blockwise_bruteforce_promotion():
    rng = np.random.default_rng(18)
    sizes, N, K = [3, 0, 2], 128, 256
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    qa, sa = bw_quantize_act_1x128(_bf(rng, (M, K)))
    qw, sw = bw_quantize_weight_128x128(_bf(rng, (G * N, K), 0.02))
    y, _ = bw_gemm_fwd(qa, sa, qw, sw, offs, N)
    A, B = e4m3_decode(qa), e4m3_decode(qw)
    grp = np.repeat(np.arange(G), sizes)
    for r, g in enumerate(grp):
        for n in range(0, N, 9):
            terms = []
            for kb in range(K // 128):
                part = math.fsum(float(A[r, k]) * float(B[g * N + n, k]) for k in range(128 * kb, 128 * kb + 128))
                terms.append(float(sa[r, kb]) * float(sw[(g * N + n) // 128, kb]) * part)
            assert math.isclose(y[r, n], math.fsum(terms), rel_tol=1e-12, abs_tol=1e-300)


def test_tolerance_checker():
    ref = np.array([1.0, -2.0, 0.0, 1000.0])
    bound = np.array([10.0, 10.0, 0.0, 1000.0])
    ok, worst, _ = check_gemm(ref + np.array([9e-5, -9e-5, 0.0, 9e-3]), ref, bound)
    assert ok and worst < 1
    ok, _, idx = check_gemm(ref + np.array([0, 0, 1e-30, 0]), ref, bound)
    assert not ok and idx == 2
    # bf16: half a bf16 ulp of (|ref| + tol) on top of the fp32 bound
    t = gemm_tolerance(np.array([1000.0]), np.array([1000.0]), "bf16")
    assert np.isclose(t[0], 1e-2 + 0.5 * 4.0)


def test_blockwise_colwise_is_act_quantiser_of_transposed_groups():
    """The 128-row column-wise blockwise quantiser of group g equals the (separately pinned) 1x128
    activation quantiser applied to the group's rows transposed and zero-padded to a multiple of
    128: zeros neither raise an amax nor change a code, and an all-zero pad tile is not stored."""
    from oracle import bw_colwise_ld_min, bw_group_columns, bw_quantize_colwise_128
    rng = np.random.default_rng(19)
    sizes, C = [0, 5, 130, 1, 300, 128, 0], 256
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    v = rng.standard_normal((M, C)) * np.where(rng.random((M, C)) < 0.01, 100.0, 1.0)
    x = f32_to_bf16_bits(v.astype(np.float32))
    ld = bw_colwise_ld_min(M, G) + 128
    qT, sT = bw_quantize_colwise_128(x, offs, ld)
    col0, nb = bw_group_columns(offs)
    assert ld == 128 * (-(-(M + 127 * G) // 128)) + 128
    used = np.zeros(ld, bool)
    for g in range(G):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        m = r1 - r0
        if m == 0:
            assert nb[g] == 0
            continue
        pad = np.zeros((128 * int(nb[g]), C), np.uint16)
        pad[:m] = x[r0:r1]
        qa, sa = bw_quantize_act_1x128(np.ascontiguousarray(pad.T))      # [C, 128 nb]
        c0 = int(col0[g])
        assert np.array_equal(qT[:, c0:c0 + m], qa[:, :m])
        assert np.array_equal(sT[:, c0 // 128:c0 // 128 + int(nb[g])], sa)
        used[c0:c0 + m] = True
    assert not qT[:, ~used].any()                      # pads and the tail are zero
    assert not sT[:, int(np.sum(nb)):].any()           # scale slots of no block are zero


def test_blockwise_wgrad_bruteforce_and_dense():
    """Blockwise wgrad against fsum triple loops with per-block promotion (tiny shapes), and for a
    single group against np.matmul of the dequantised column-wise operands."""
    from oracle import bw_colwise_ld_min, bw_gemm_wgrad, bw_group_columns, bw_quantize_colwise_128
    rng = np.random.default_rng(20)
    sizes, N, K = [3, 0, 130], 128, 128
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    ld = bw_colwise_ld_min(M, G)
    qd, sd = bw_quantize_colwise_128(_bf(rng, (M, N)), offs, ld)
    qx, sx = bw_quantize_colwise_128(_bf(rng, (M, K)), offs, ld)
    dw, bnd = bw_gemm_wgrad(qd, sd, qx, sx, offs, N, K)
    assert not dw[1].any() and not bnd[1].any()        # empty expert: zero gradient
    A, B = e4m3_decode(qd), e4m3_decode(qx)
    col0, nb = bw_group_columns(offs)
    for g in (0, 2):
        c0, m = int(col0[g]), sizes[g]
        for n in range(0, N, 17):
            for k in range(0, K, 23):
                terms = []
                for b in range(int(nb[g])):
                    js = range(c0 + 128 * b, min(c0 + 128 * b + 128, c0 + m))
                    part = math.fsum(float(A[n, j]) * float(B[k, j]) for j in js)
                    terms.append(float(sd[n, c0 // 128 + b]) * float(sx[k, c0 // 128 + b]) * part)
                assert math.isclose(dw[g, n, k], math.fsum(terms), rel_tol=1e-12, abs_tol=1e-300)
    # one group of 256 tokens: the dense product of the dequantised operands
    offs1 = np.array([0, 256])
    ld1 = bw_colwise_ld_min(256, 1)
    qd1, sd1 = bw_quantize_colwise_128(_bf(rng, (256, N)), offs1, ld1)
    qx1, sx1 = bw_quantize_colwise_128(_bf(rng, (256, K)), offs1, ld1)
    dw1, bnd1 = bw_gemm_wgrad(qd1, sd1, qx1, sx1, offs1, N, K)
    Dd = e4m3_decode(qd1[:, :256]) * np.repeat(sd1[:, :2].astype(np.float64), 128, axis=1)
    Dx = e4m3_decode(qx1[:, :256]) * np.repeat(sx1[:, :2].astype(np.float64), 128, axis=1)
    # products of two fp32 scales and two E4M3 codes need up to 56 bits, so both sides round in
    # float64: compare relative to sum |a b|
    assert np.all(np.abs(dw1[0] - np.matmul(Dd, Dx.T)) <= 1e-12 * bnd1[0])
