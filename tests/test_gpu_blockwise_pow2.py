"""GPU parity of the power-of-two blockwise mode: the three quantisers bit-exact against the oracle
(every finite bf16 magnitude as a tile's amax, ragged experts, outliers, zero tiles), and the blockwise
GEMMs on their outputs within 1e-5 * sum|ab|."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host, random_bf16, require_gpu, same_bytes
from workloads import f32_to_bf16_bits, routing_offsets

pytestmark = pytest.mark.gpu


def _equal(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what} mismatch at {bad[:5]}: gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]}"


def test_act_every_bf16_magnitude_as_tile_amax():
    m = require_gpu()
    rng = np.random.default_rng(60)
    mags = np.arange(1, 0x7F80, dtype=np.uint32)                  # every finite non-zero magnitude
    amax = (mags << 16).view(np.float32)
    u = rng.uniform(-1.0, 1.0, (len(mags), 128)).astype(np.float32)
    v = (u * amax[:, None]).astype(np.float32)
    v[:, 0] = amax                                               # the tile's maximum, exactly
    v[1::2, 0] *= -1                                             # and negative in every other tile
    x = f32_to_bf16_bits(v)
    q, s = m.fp8bw_quantize_act_1x128(dev(x), pow2=True)
    qo, so = oracle.bw_quantize_act_1x128(x, pow2=True)
    _equal(host(s), so, "scale")
    _equal(host(q), qo, "code")


def test_quantisers_random_shapes_and_zero_tiles():
    m = require_gpu()
    rng = np.random.default_rng(61)
    for R, C in ((1, 128), (37, 384), (300, 1024)):
        x = random_bf16(rng, (R, C), outlier_frac=0.01, outlier_mult=1e4)
        x[0, :128] = 0                                           # an all-zero tile -> scale 1
        q, s = m.fp8bw_quantize_act_1x128(dev(x), pow2=True)
        qo, so = oracle.bw_quantize_act_1x128(x, pow2=True)
        _equal(host(s), so, "act scale")
        _equal(host(q), qo, "act code")
    for R, C in ((128, 128), (512, 384)):
        w = random_bf16(rng, (R, C), std=0.02, outlier_frac=0.001)
        w[:128, :128] = 0
        q, s, qT = m.fp8bw_quantize_weight_128x128(dev(w), transposed=True, pow2=True)
        qo, so = oracle.bw_quantize_weight_128x128(w, pow2=True)
        _equal(host(s), so, "weight scale")
        _equal(host(q), qo, "weight code")
        _equal(host(qT), qo.T, "transposed weight code")


def test_colwise_ragged_groups():
    m = require_gpu()
    rng = np.random.default_rng(62)
    sizes = [0, 5, 130, 1, 300, 128, 0]
    offs = routing_offsets(sizes)
    M = int(offs[-1])
    x = random_bf16(rng, (M, 384), outlier_frac=0.01, outlier_mult=1000.0)
    x[5:135, :128] = 0                                           # an all-zero block: scale 1
    for extra in (0, 128):
        ld = oracle.bw_colwise_ld_min(M, len(sizes)) + extra
        qT, sT = m.fp8bw_quantize_colwise_128(dev(x), dev(offs), ld=ld, pow2=True)
        qo, so = oracle.bw_quantize_colwise_128(x, offs, ld, pow2=True)
        _equal(host(sT), so, "colwise scale")
        _equal(host(qT), qo, "colwise code")


def test_gemms_on_power_of_two_operands():
    m = require_gpu()
    rng = np.random.default_rng(63)
    for sizes, N, K in (([0, 5, 130, 1, 60], 256, 1024), ([129, 0, 17], 128, 256)):
        offs = routing_offsets(sizes)
        M, G = int(offs[-1]), len(sizes)
        x = random_bf16(rng, (M, K), outlier_frac=0.001)
        w = random_bf16(rng, (G * N, K), std=0.02, outlier_frac=0.001)
        dy = random_bf16(rng, (M, N))
        od = dev(offs)
        qx, sx = m.fp8bw_quantize_act_1x128(dev(x), pow2=True)
        qw, sw, qwT = m.fp8bw_quantize_weight_128x128(dev(w), transposed=True, pow2=True)
        same_bytes((host(qx), host(sx)), oracle.bw_quantize_act_1x128(x, pow2=True), "pow2 X")
        wq = oracle.bw_quantize_weight_128x128(w, pow2=True)
        same_bytes((host(qw), host(sw), host(qwT)), (wq[0], wq[1], wq[0].T), "pow2 W")
        y = m.fp8bw_grouped_gemm_fwd(qx, sx, qw, sw, od, N)
        ref, bnd = oracle.bw_gemm_fwd(host(qx), host(sx), host(qw), host(sw), offs, N)
        ok, worst, _ = oracle.check_gemm(host(y), ref, bnd, "f32")
        assert ok, f"fwd worst err/tol {worst}"
        qd, sd = m.fp8bw_quantize_act_1x128(dev(dy), pow2=True)
        same_bytes((host(qd), host(sd)), oracle.bw_quantize_act_1x128(dy, pow2=True), "pow2 dY")
        dx = m.fp8bw_grouped_gemm_dgrad(qd, sd, qwT, sw, od, K)
        ref, bnd = oracle.bw_gemm_dgrad(host(qd), host(sd), host(qw), host(sw), offs, N, K)
        ok, worst, _ = oracle.check_gemm(host(dx), ref, bnd, "f32")
        assert ok, f"dgrad worst err/tol {worst}"
        ld = oracle.bw_colwise_ld_min(M, G)
        qdT, sdT = m.fp8bw_quantize_colwise_128(dev(dy), od, ld=ld, pow2=True)
        qxT, sxT = m.fp8bw_quantize_colwise_128(dev(x), od, ld=ld, pow2=True)
        same_bytes((host(qdT), host(sdT)), oracle.bw_quantize_colwise_128(dy, offs, ld, pow2=True), "pow2 dY 128-token")
        same_bytes((host(qxT), host(sxT)), oracle.bw_quantize_colwise_128(x, offs, ld, pow2=True), "pow2 X 128-token")
        dw = m.fp8bw_grouped_gemm_wgrad(qdT, sdT, qxT, sxT, od, M, "f32")
        ref, bnd = oracle.bw_gemm_wgrad(host(qdT), host(sdT), host(qxT), host(sxT), offs, N, K)
        ok, worst, _ = oracle.check_gemm(host(dw), ref, bnd, "f32")
        assert ok, f"wgrad worst err/tol {worst}"
        torch.cuda.synchronize()


@pytest.mark.parametrize("fast", [False, True])
def test_pow2_gemms_on_the_mx_kernel(fast):
    """fp8bw_grouped_gemm_{fwd,dgrad,wgrad}_pow2: power-of-two blockwise scales folded into the operands
    on the MX kernel, against the oracle's promoted blockwise products (within 1e-5 sum|ab|; the FP8
    feed within its 2^-10 bound), on ragged experts (empty, 1, 17, 129 rows) and both output dtypes;
    the weight gradient also with a padded leading dimension (empty experts give zeros)."""
    m = require_gpu()
    rng = np.random.default_rng(64)
    rel = 2.0 ** -10 if fast else oracle.gemm.REL_TOL
    for sizes, N, K in (([0, 5, 130, 1, 60], 256, 1024), ([129, 0, 17], 128, 256),
                        ([700, 0, 129, 1, 513, 64], 384, 768)):
        offs = routing_offsets(sizes)
        M, G = int(offs[-1]), len(sizes)
        x = random_bf16(rng, (M, K), outlier_frac=0.001, outlier_mult=1000.0)
        w = random_bf16(rng, (G * N, K), std=0.02, outlier_frac=0.001)
        dy = random_bf16(rng, (M, N), outlier_frac=0.001)
        od = dev(offs)
        qx, sx = m.fp8bw_quantize_act_1x128(dev(x), pow2=True)
        qw, sw, qwT = m.fp8bw_quantize_weight_128x128(dev(w), transposed=True, pow2=True)
        qd, sd = m.fp8bw_quantize_act_1x128(dev(dy), pow2=True)
        xq = oracle.bw_quantize_act_1x128(x, pow2=True)
        wq = oracle.bw_quantize_weight_128x128(w, pow2=True)
        dq = oracle.bw_quantize_act_1x128(dy, pow2=True)
        same_bytes((host(qx), host(sx), host(qw), host(sw), host(qwT), host(qd), host(sd)),
                   (xq[0], xq[1], wq[0], wq[1], wq[0].T, dq[0], dq[1]), "pow2 operands")
        for dt in ("f32", "bf16"):
            y = m.fp8bw_grouped_gemm_fwd_pow2(qx, sx, qw, sw, od, N, dt, fast=fast)
            ref, bnd = oracle.bw_gemm_fwd(xq[0], xq[1], wq[0], wq[1], offs, N)
            got = host(y)
            got = (got.astype(np.uint32) << 16).view(np.float32) if dt == "bf16" else got
            ok, worst, _ = oracle.check_gemm(got, ref, bnd, dt, rel=rel)
            assert ok, f"fwd_pow2 {sizes} {dt}: worst err/tol {worst:.3g}"
            dx = m.fp8bw_grouped_gemm_dgrad_pow2(qd, sd, qwT, sw, od, K, dt, fast=fast)
            ref, bnd = oracle.bw_gemm_dgrad(dq[0], dq[1], wq[0], wq[1], offs, N, K)
            got = host(dx)
            got = (got.astype(np.uint32) << 16).view(np.float32) if dt == "bf16" else got
            ok, worst, _ = oracle.check_gemm(got, ref, bnd, dt, rel=rel)
            assert ok, f"dgrad_pow2 {sizes} {dt}: worst err/tol {worst:.3g}"
        for extra in (0, 256):
            ld = oracle.bw_colwise_ld_min(M, G) + extra
            qdT, sdT = m.fp8bw_quantize_colwise_128(dev(dy), od, ld=ld, pow2=True)
            qxT, sxT = m.fp8bw_quantize_colwise_128(dev(x), od, ld=ld, pow2=True)
            cd = oracle.bw_quantize_colwise_128(dy, offs, ld, pow2=True)
            cx = oracle.bw_quantize_colwise_128(x, offs, ld, pow2=True)
            same_bytes((host(qdT), host(sdT), host(qxT), host(sxT)), (cd[0], cd[1], cx[0], cx[1]), "pow2 128-token")
            dw = torch.full((G, N, K), float("nan"), dtype=torch.float32, device="cuda")
            m.fp8bw_grouped_gemm_wgrad_pow2(qdT, sdT, qxT, sxT, od, M, "f32", dw=dw, fast=fast)
            ref, bnd = oracle.bw_gemm_wgrad(cd[0], cd[1], cx[0], cx[1], offs, N, K)
            ok, worst, _ = oracle.check_gemm(host(dw), ref, bnd, "f32", rel=rel)
            assert ok, f"wgrad_pow2 {sizes} ld {ld}: worst err/tol {worst:.3g}"
        torch.cuda.synchronize()
