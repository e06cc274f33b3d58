"""GPU parity of the MXFP4 path (E2M1 codes two per byte, E8M0 per 32): quantisers bit-exact against
the oracle, GEMMs (block-scaled FP4 MFMA) within 1e-5 * sum|a b| of the oracle evaluated on the GPU's
own quantised operands."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_rows, dev, host, random_bf16, require_gpu, same_bytes
from test_gpu_gemm import _check, _gpu_out, _rand_layer
from workloads import f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


def _finite_bf16_patterns():
    b = np.arange(65536, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def _rowwise_equal(m, x):
    q, s = m.mxfp4_quantize_rowwise(dev(x))
    qo, so = oracle.mxfp4_quantize_rowwise(x)
    assert np.array_equal(host(s), so), f"scale mismatch at {np.argwhere(host(s) != so)[:5]}"
    bad = np.argwhere(host(q) != qo)
    assert bad.size == 0, f"code mismatch at {bad[:5]}"


def test_rowwise_exhaustive_bf16():
    """Every finite bf16 pattern as a block maximum, and below fixed maxima."""
    m = require_gpu()
    p = _finite_bf16_patterns()
    x = np.zeros((len(p), 32), np.uint16)
    x[:, 0] = p
    x[:, 1] = p ^ 0x8000
    _rowwise_equal(m, x)
    for amax in (1.0, 6.0, 2.0 ** -100, 2.0 ** 60):
        v = (p.astype(np.uint32) << 16).view(np.float32)
        sel = p[np.abs(v) <= amax]
        n = (len(sel) + 30) // 31
        x = np.zeros((n, 32), np.uint16)
        flat = np.zeros(n * 31, np.uint16)
        flat[:len(sel)] = sel
        x[:, :31] = flat.reshape(n, 31)
        x[:, 31] = f32_to_bf16_bits(np.array([amax], np.float32))[0]
        _rowwise_equal(m, x)


def test_rowwise_random_shapes():
    m = require_gpu()
    rng = np.random.default_rng(40)
    for R, C in ((1, 32), (3, 96), (257, 512), (1000, 2048)):
        _rowwise_equal(m, random_bf16(rng, (R, C), outlier_frac=0.01, outlier_mult=1000.0))


def test_colwise_ragged_and_weight_layout():
    m = require_gpu()
    rng = np.random.default_rng(41)
    sizes = [0, 5, 130, 1, 60, 33, 0]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offs[-1])
    for C in (32, 288, 512):
        x = random_bf16(rng, (M, C), outlier_frac=0.01, outlier_mult=1000.0)
        for extra in (0, 64):
            ld = oracle.mx_colwise_ld_min(M, len(sizes)) + extra
            qT, sT = m.mxfp4_quantize_colwise(dev(x), dev(offs), ld=ld)
            qo, so = oracle.mxfp4_quantize_colwise(x, offs, ld)
            assert np.array_equal(host(sT), so) and np.array_equal(host(qT), qo)
    w = random_bf16(rng, (4 * 256, 512), std=0.02)
    qT, sT = m.mxfp4_quantize_colwise(dev(w), None, ld=1024)
    qo, so = oracle.mxfp4_quantize_colwise(w, None, 1024)
    assert np.array_equal(host(sT), so) and np.array_equal(host(qT), qo)


def _fp4_layer_check(m, L, dt, rows=None, groups=None, n_idx=None, k_idx=None, extra=0):
    offs = dev(L.offs)
    w2 = L.w.reshape(-1, L.K)
    x, w, dy = dev(L.x), dev(w2), dev(L.dy)
    worst = {}
    r_chk = check_rows(L.M, rows, cap=1 << 30)
    w_chk = check_rows(L.G * L.N, seed=73)
    qx, sx = m.mxfp4_quantize_rowwise(x)
    qw, sw = m.mxfp4_quantize_rowwise(w)
    same_bytes((host(qx)[r_chk], host(sx)[r_chk]), oracle.mxfp4_quantize_rowwise(L.x[r_chk]), "E2M1 X row-wise")
    same_bytes((host(qw)[w_chk], host(sw)[w_chk]), oracle.mxfp4_quantize_rowwise(w2[w_chk]), "E2M1 W row-wise")
    y = m.mxfp4_grouped_gemm_fwd(qx, sx, qw, sw, offs, L.N, dt)
    ref, bnd = oracle.mxfp4_gemm_fwd(host(qx), host(sx), host(qw), host(sw), L.offs, L.N, rows=rows)
    got = _gpu_out(y) if rows is None else _gpu_out(y)[rows]
    worst["fwd"] = _check(got, ref, bnd, dt, "fp4 fwd")
    qd, sd = m.mxfp4_quantize_rowwise(dy)
    qwT, swT = m.mxfp4_quantize_colwise(w, None, ld=L.G * L.N)
    k_chk = check_rows(L.K, seed=74, cap=32)
    same_bytes((host(qd)[r_chk], host(sd)[r_chk]), oracle.mxfp4_quantize_rowwise(L.dy[r_chk]), "E2M1 dY row-wise")
    same_bytes((host(qwT)[k_chk], host(swT)[k_chk]), oracle.mxfp4_quantize_colwise(w2[:, k_chk], None, L.G * L.N),
               "E2M1 W column-wise")
    dx = m.mxfp4_grouped_gemm_dgrad(qd, sd, qwT, swT, offs, L.K, dt)
    ref, bnd = oracle.mxfp4_gemm_dgrad(host(qd), host(sd), host(qwT), host(swT), L.offs, L.N, L.K, rows=rows)
    got = _gpu_out(dx) if rows is None else _gpu_out(dx)[rows]
    worst["dgrad"] = _check(got, ref, bnd, dt, "fp4 dgrad")
    # the pitch the benchmark uses (padded off slow byte pitches), or the minimum plus `extra` elements
    ld = m.mxfp4_colwise_ld(L.M, L.G) + extra
    assert ld >= oracle.mx_colwise_ld_min(L.M, L.G)
    qdT, sdT = m.mxfp4_quantize_colwise(dy, offs, ld=ld)
    qxT, sxT = m.mxfp4_quantize_colwise(x, offs, ld=ld)
    dw = m.mxfp4_grouped_gemm_wgrad(qdT, sdT, qxT, sxT, offs, L.M, dt)
    n_chk, k_chk = check_rows(L.N, n_idx, cap=1 << 30), check_rows(L.K, k_idx, cap=1 << 30)
    same_bytes((host(qdT)[n_chk], host(sdT)[n_chk]), oracle.mxfp4_quantize_colwise(L.dy[:, n_chk], L.offs, ld),
               "E2M1 dY column-wise")
    same_bytes((host(qxT)[k_chk], host(sxT)[k_chk]), oracle.mxfp4_quantize_colwise(L.x[:, k_chk], L.offs, ld),
               "E2M1 X column-wise")
    ref, bnd = oracle.mxfp4_gemm_wgrad(host(qdT), host(sdT), host(qxT), host(sxT), L.offs, L.N, L.K,
                                       groups=groups, n_idx=n_idx, k_idx=k_idx)
    got = _gpu_out(dw)
    if groups is not None:
        got = got[np.ix_(groups, n_idx, k_idx)]
    worst["wgrad"] = _check(got, ref, bnd, dt, "fp4 wgrad")
    return worst


def test_gemms_ragged_groups():
    """Ragged experts (empty, 1, 5, 130, 300 rows; wgrad contraction lengths not a multiple of the
    256-element stage), fp32 and bf16 outputs."""
    m = require_gpu()
    rng = np.random.default_rng(42)
    for sizes, N, K in (([0, 5, 130, 1, 300], 256, 512), ([257, 0, 17], 512, 256)):
        L = _rand_layer(rng, sizes, N, K, outliers=0.001)
        for dt in ("f32", "bf16"):
            print("fp4", sizes, dt, _fp4_layer_check(m, L, dt))
    # a padded leading dimension (2048 elements = 1 KiB of E2M1 codes per qT row)
    L = _rand_layer(rng, [0, 5, 130, 1, 300], 256, 512, outliers=0.001)
    print("fp4 padded ld", _fp4_layer_check(m, L, "f32", extra=2048))


def test_wgrad_at_two_scale_pitches():
    """MXFP4 weight gradient (its scale rows are always gathered through registers) at a scale pitch of
    unaligned rows (ld / 32 not a multiple of 4) and at the recommended pitch (aligned rows): experts
    start at blocks of every residue mod 4, with stages of 1 to 8 valid blocks."""
    m = require_gpu()
    rng = np.random.default_rng(43)
    sizes = [0, 70, 300, 40, 128, 200, 5, 150, 33, 180]
    L = _rand_layer(rng, sizes, 256, 512, outliers=0.002)
    offs = dev(L.offs)
    x, dy = dev(L.x), dev(L.dy)
    ld_min = oracle.mx_colwise_ld_min(L.M, L.G)
    assert (ld_min // 32) % 4 != 0
    for ld in (ld_min, m.mxfp4_colwise_ld(L.M, L.G)):
        qdT, sdT = m.mxfp4_quantize_colwise(dy, offs, ld=ld)
        qxT, sxT = m.mxfp4_quantize_colwise(x, offs, ld=ld)
        same_bytes((host(qdT), host(sdT)), oracle.mxfp4_quantize_colwise(L.dy, L.offs, ld), "E2M1 dY column-wise")
        same_bytes((host(qxT), host(sxT)), oracle.mxfp4_quantize_colwise(L.x, L.offs, ld), "E2M1 X column-wise")
        ref, bnd = oracle.mxfp4_gemm_wgrad(host(qdT), host(sdT), host(qxT), host(sxT), L.offs, L.N, L.K)
        for dt in ("f32", "bf16"):
            dw = m.mxfp4_grouped_gemm_wgrad(qdT, sdT, qxT, sxT, offs, L.M, dt)
            print("fp4 wgrad ld", ld, dt, _check(_gpu_out(dw), ref, bnd, dt, f"fp4 wgrad ld={ld} {dt}"))


def test_run_of_mixed_magnitudes_is_exact():
    """Products 36 and 0.25 (6 x 6 and 0.5 x 0.5) side by side in every 32-block, and blocks whose
    scales differ by up to 2^+-4: all terms are multiples of 2^-6 below 2^18, so every partial sum is
    exact in fp32 and the result must equal the oracle bit for bit."""
    m = require_gpu()
    rng = np.random.default_rng(43)
    M, N, K = 64, 256, 256
    offs = np.array([0, M], np.int32)
    xv = np.where(rng.random((M, K)) < 0.5, 6.0, 0.5) * np.where(rng.random((M, K)) < 0.5, -1, 1)
    wv = np.where(rng.random((N, K)) < 0.5, 6.0, 0.5)
    blk = rng.integers(-4, 5, K // 32)
    xv = xv * np.repeat(2.0 ** blk, 32)[None, :]
    x = f32_to_bf16_bits(xv.astype(np.float32))
    w = f32_to_bf16_bits(wv.astype(np.float32))
    qx, sx = m.mxfp4_quantize_rowwise(dev(x))
    qw, sw = m.mxfp4_quantize_rowwise(dev(w))
    same_bytes((host(qx), host(sx)), oracle.mxfp4_quantize_rowwise(x), "E2M1 X row-wise")
    same_bytes((host(qw), host(sw)), oracle.mxfp4_quantize_rowwise(w), "E2M1 W row-wise")
    y = m.mxfp4_grouped_gemm_fwd(qx, sx, qw, sw, dev(offs), N, "f32")
    ref, _ = oracle.mxfp4_gemm_fwd(host(qx), host(sx), host(qw), host(sw), offs, N)
    assert np.array_equal(_gpu_out(y), ref)


def test_full_size_sampled():
    """DeepSeek-V3-671B expert shard (N, K multiples of 256): full launches, sampled rows / experts."""
    m = require_gpu()
    wl = make_workload("dsv3_671b_shard")
    rng = np.random.default_rng(44)
    for lay in wl.layers:
        rows = np.unique(np.concatenate([[0, lay.M - 1], rng.choice(lay.M, 48, replace=False)]))
        groups = np.unique(np.concatenate([np.argsort(np.diff(lay.offs))[:2], [int(np.argmax(np.diff(lay.offs)))]]))
        n_idx = np.unique(rng.choice(lay.N, 16, replace=False))
        k_idx = np.unique(rng.choice(lay.K, 16, replace=False))
        print(lay.name, _fp4_layer_check(m, lay, "f32", rows=rows, groups=groups, n_idx=n_idx, k_idx=k_idx))
        torch.cuda.empty_cache()
