"""The 128-byte tiled layouts on the GPU (column-wise codes and every scale buffer tiled).

Quantiser outputs are compared byte for byte with the oracle's quantisation permuted by
oracle.mx_colwise_tiled and oracle.mx_scales_tiled (the layout's stated contract); the GEMMs that read
tiled operands must give results bit-identical to the row-major entry points on the same data and lie
within the oracle's bound; the gated forward's tiled H is compared with the oracle's quantisation of
the kernel's H.
Output buffers are pre-filled with 0xAB so that every byte the contract defines must be written."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host, random_bf16, require_gpu, same_bytes
from workloads import make_workload, random_offsets, routing_offsets

pytestmark = pytest.mark.gpu

FAST_REL = 2.0 ** -10          # the FP8 feed's bound (see test_gpu_gemm)


def _ld128(n):
    return 128 * ((n + 127) // 128)


def _filled(shape, dtype=torch.uint8):
    return torch.full(shape, 0xAB, dtype=dtype, device="cuda")


def _untile(t):
    """[ld/128, C, 128] tiled bytes (or [ld/128, C, 4] tiled scales) -> the row-major [C, ld] copy."""
    a = host(t)
    T, C, W = a.shape
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(C, T * W))


def _tiles(qo, so):
    """The oracle's row-major column-wise copy in the tiled layout (codes and scales)."""
    return oracle.mx_colwise_tiled(qo), oracle.mx_scales_tiled(so)


def _colwise_tiled_equal(m, x, offs, ld):
    R, C = x.shape
    qT, sT = _filled((ld // 128, C, 128)), _filled((ld // 128, C, 4))
    m.mx_quantize_colwise_tiled(dev(x), None if offs is None else dev(np.asarray(offs, np.int32)), ld=ld, qT=qT,
                                sT=sT)
    qo, so = oracle.mx_quantize_colwise(x, offs, ld)
    same_bytes((host(qT), host(sT)), _tiles(qo, so), f"tiled column-wise {R}x{C} ld {ld}")


def test_colwise_tiled_ragged_groups():
    m = require_gpu()
    rng = np.random.default_rng(81)
    for sizes, C in (([17, 0, 33, 1, 70], 64), ([0, 0, 5], 32), ([128], 96), ([31, 32, 33, 0, 64, 1], 160),
                     ([300, 2, 129], 512)):
        offs = routing_offsets(sizes)
        M = int(offs[-1])
        x = random_bf16(rng, (M, C), outlier_frac=0.02)
        ld = _ld128(oracle.mx_colwise_ld_min(M, len(sizes)))
        _colwise_tiled_equal(m, x, offs, ld)
        _colwise_tiled_equal(m, x, offs, ld + 256)          # extra tail tiles are zero
    offs = random_offsets(rng, 3000, 37)
    _colwise_tiled_equal(m, random_bf16(rng, (3000, 128), outlier_frac=0.001), offs,
                         _ld128(oracle.mx_colwise_ld_min(3000, 37)))
    # one group (the weight copy of the dgrad), a row count that is not a multiple of 128
    w = random_bf16(rng, (4 * 96 + 40, 256), std=0.02)
    _colwise_tiled_equal(m, w, None, _ld128(w.shape[0]))


def _dual_tiled_equal(m, x, offs, ld, row_idx=None):
    R = x.shape[0] if row_idx is None else len(row_idx)
    C = x.shape[1]
    q, s = _filled((R, C)), _filled((C // 128, R, 4))
    qT, sT = _filled((ld // 128, C, 128)), _filled((ld // 128, C, 4))
    m.mx_quantize_dual_tiled(dev(x), None if offs is None else dev(offs), ld=ld,
                             row_idx=None if row_idx is None else dev(row_idx), q=q, s=s, qT=qT, sT=sT)
    ro = oracle.mx_quantize_dual(x, offs, ld, row_idx)
    same_bytes((host(q), host(s), host(qT), host(sT)), (ro[0], oracle.mx_scales_tiled(ro[1])) + _tiles(ro[2], ro[3]),
               f"tiled dual {R}x{C} ld {ld}")


def test_rowwise_tiled():
    m = require_gpu()
    rng = np.random.default_rng(86)
    for R, C in ((1, 128), (37, 256), (300, 384), (1000, 1152)):
        x = random_bf16(rng, (R, C), outlier_frac=0.01, outlier_mult=1000.0)
        q, s = _filled((R, C)), _filled((C // 128, R, 4))
        m.mx_quantize_rowwise_tiled(dev(x), q=q, s=s)
        qo, so = oracle.mx_quantize_rowwise(x)
        same_bytes((host(q), host(s)), (qo, oracle.mx_scales_tiled(so)), f"tiled row-wise {R}x{C}")


def test_dual_tiled_ragged_groups_partial_windows_and_gather():
    m = require_gpu()
    rng = np.random.default_rng(82)
    sizes = [0, 5, 130, 1, 60, 33, 0]
    offs = routing_offsets(sizes)
    M = int(offs[-1])
    for C in (128, 384, 512, 1152):                 # 384 and 1152: a last window of 128 columns
        x = random_bf16(rng, (M, C), outlier_frac=0.01, outlier_mult=1000.0)
        ld = _ld128(oracle.mx_colwise_ld_min(M, len(sizes)))
        _dual_tiled_equal(m, x, offs, ld)
        _dual_tiled_equal(m, x, offs, ld + 128)
    x = random_bf16(rng, (3 * 128 + 7, 640), std=0.02)
    _dual_tiled_equal(m, x, None, _ld128(x.shape[0]))
    # routed rows gathered by index (top-2), two indices out of range (clamped)
    T, C, G = 300, 384, 5
    x = random_bf16(rng, (T, C), outlier_frac=0.01)
    experts = np.stack([rng.choice(G, 2, replace=False) for _ in range(T)])
    tok = np.repeat(np.arange(T), 2)
    order = np.argsort(experts.reshape(-1), kind="stable")
    row_idx = tok[order].astype(np.int32)
    row_idx[3], row_idx[9] = -1, T + 7
    offs = np.concatenate([[0], np.cumsum(np.bincount(experts.reshape(-1), minlength=G))]).astype(np.int32)
    _dual_tiled_equal(m, x, offs, _ld128(oracle.mx_colwise_ld_min(2 * T, G)), row_idx)


def test_dual_tiled_full_size_sampled():
    """DeepSeek-V3-671B shard, gate+up X [65536, 7168] at the benchmark's pitch: sampled rows (row-wise)
    and columns (column-wise, read back out of the tiles) against the oracle."""
    m = require_gpu()
    lay = make_workload("dsv3_671b_shard", layers=["gate_up"]).layers[0]
    rng = np.random.default_rng(83)
    rows = np.concatenate([[0, lay.M - 1], rng.choice(lay.M, 200, replace=False)])
    cols = np.unique(np.concatenate([[0, lay.K - 1], rng.choice(lay.K, 24, replace=False)]))
    ld = m.mx_colwise_ld(lay.M, lay.G)
    assert ld % 128 == 0
    q, s, qT, sT = m.mx_quantize_dual_tiled(dev(lay.x), dev(lay.offs), ld=ld)
    same_bytes((host(q[rows]), _untile(s[:, rows, :])), oracle.mx_quantize_rowwise(lay.x[rows]),
               "dual tiled, row-wise")
    qo, so = oracle.mx_quantize_colwise(np.ascontiguousarray(lay.x[:, cols]), lay.offs, ld)
    same_bytes((_untile(qT[:, cols, :]), _untile(sT[:, cols, :])), (qo, so), "dual tiled, column-wise")
    del q, s, qT, sT
    torch.cuda.empty_cache()


def _layer(rng, sizes, N, K):
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    return (offs, random_bf16(rng, (M, K), outlier_frac=0.001), random_bf16(rng, (G * N, K), 0.05),
            random_bf16(rng, (M, N), outlier_frac=0.001))


@pytest.mark.parametrize("fast", [False, True])
def test_gemms_on_tiled_operands(fast):
    """fwd, dgrad and wgrad from tiled operands: bit-identical to the row-major entry points, and
    within the oracle's bound on the oracle's own quantisation (the tiled bytes checked first)."""
    m = require_gpu()
    rng = np.random.default_rng(84)
    rel = FAST_REL if fast else oracle.gemm.REL_TOL
    for sizes, N, K in (([0, 5, 130, 1, 300, 33], 256, 384), ([257, 0, 17, 512], 384, 256), ([700], 128, 128)):
        offs, x, w, dy = _layer(rng, sizes, N, K)
        M, G = int(offs[-1]), len(sizes)
        offs_d = dev(offs)
        # forward: row-wise X and W with tiled scales
        qx, sx = m.mx_quantize_rowwise(dev(x))
        qw, sw = m.mx_quantize_rowwise(dev(w))
        qxt, sxt = m.mx_quantize_rowwise_tiled(dev(x))
        qwt, swt = m.mx_quantize_rowwise_tiled(dev(w))
        xo, wo = oracle.mx_quantize_rowwise(x), oracle.mx_quantize_rowwise(w)
        same_bytes((host(qxt), host(sxt), host(qwt), host(swt)),
                   (xo[0], oracle.mx_scales_tiled(xo[1]), wo[0], oracle.mx_scales_tiled(wo[1])), "X, W row-wise tiled")
        y = m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs_d, N, "f32", fast=fast)
        yt = m.mx_grouped_gemm_fwd_tiled(qxt, sxt, qwt, swt, offs_d, N, "f32", fast=fast)
        assert torch.equal(y, yt), "fwd: tiled scales give other bits than the row-major ones"
        ref, bnd = oracle.mx_gemm_fwd(*xo, *wo, offs, N)
        ok, worst, _ = oracle.check_gemm(host(yt).astype(np.float64), ref, bnd, "f32", rel=rel)
        assert ok, f"fwd tiled: worst err/tol {worst:.3g}"
        # dgrad: dY row-wise (tiled scales), W column-wise [K, ldw] (ldw padded past G*N)
        qdy, sdy = m.mx_quantize_rowwise(dev(dy))
        qdyr, sdyt = m.mx_quantize_rowwise_tiled(dev(dy))
        same_bytes((host(qdyr), host(sdyt)), (host(qdy), oracle.mx_scales_tiled(host(sdy))), "dY row-wise tiled")
        ldw = _ld128(G * N) + 128
        qwT, swT = m.mx_quantize_colwise(dev(w), None, ld=ldw)
        qwTt, swTt = m.mx_quantize_colwise_tiled(dev(w), None, ld=ldw)
        same_bytes((host(qwTt), host(swTt)), _tiles(host(qwT), host(swT)), "W tiled vs row-major")
        dx = m.mx_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs_d, K, "f32", fast=fast)
        dxt = m.mx_grouped_gemm_dgrad_tiled(qdyr, sdyt, qwTt, swTt, offs_d, K, "f32", fast=fast)
        assert torch.equal(dx, dxt), "dgrad: tiled operand gives other bits than the row-major one"
        qo, so = oracle.mx_quantize_colwise(w, None, ldw)
        same_bytes((host(qwTt), host(swTt)), _tiles(qo, so), "W tiled")
        ref, bnd = oracle.mx_gemm_dgrad(*oracle.mx_quantize_rowwise(dy), qo, so, offs, N, K)
        ok, worst, _ = oracle.check_gemm(host(dxt).astype(np.float64), ref, bnd, "f32", rel=rel)
        assert ok, f"dgrad tiled: worst err/tol {worst:.3g}"
        # wgrad: dY and X column-wise, the recommended pitch
        ld = m.mx_colwise_ld(M, G)
        qdyT, sdyT = m.mx_quantize_colwise(dev(dy), offs_d, ld=ld)
        qxT, sxT = m.mx_quantize_colwise(dev(x), offs_d, ld=ld)
        qdyTt, sdyTt = m.mx_quantize_colwise_tiled(dev(dy), offs_d, ld=ld)
        qxTt, sxTt = m.mx_quantize_colwise_tiled(dev(x), offs_d, ld=ld)
        for bf16 in (False, True):
            dt = "bf16" if bf16 else "f32"
            dw = m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs_d, M, dt, fast=fast)
            dwt = m.mx_grouped_gemm_wgrad_tiled(qdyTt, sdyTt, qxTt, sxTt, offs_d, M, dt, fast=fast)
            assert torch.equal(dw, dwt), f"wgrad ({dt}): tiled operands give other bits than the row-major ones"
        qa, sa = oracle.mx_quantize_colwise(dy, offs, ld)
        qb, sb = oracle.mx_quantize_colwise(x, offs, ld)
        same_bytes((host(qdyTt), host(sdyTt), host(qxTt), host(sxTt)), _tiles(qa, sa) + _tiles(qb, sb),
                   "dY, X tiled")
        ref, bnd = oracle.mx_gemm_wgrad(qa, sa, qb, sb, offs, N, K)
        dw = m.mx_grouped_gemm_wgrad_tiled(qdyTt, sdyTt, qxTt, sxTt, offs_d, M, "f32", fast=fast)
        ok, worst, _ = oracle.check_gemm(host(dw).astype(np.float64), ref, bnd, "f32", rel=rel)
        assert ok, f"wgrad tiled: worst err/tol {worst:.3g}"


def test_gemms_on_tiled_operands_full_size():
    """DeepSeek-V3-671B shard gate+up fwd, dgrad and wgrad at full size: the tiled-operand launches give
    the row-major launches' bits exactly, on every element."""
    m = require_gpu()
    lay = make_workload("dsv3_671b_shard", layers=["gate_up"]).layers[0]
    G, M, N, K = lay.G, lay.M, lay.N, lay.K
    offs = dev(lay.offs)
    x, dy, w = dev(lay.x), dev(lay.dy), dev(lay.w.reshape(G * N, K))
    qx, sx = m.mx_quantize_rowwise(x)
    qw, sw = m.mx_quantize_rowwise(w)
    a = m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs, N, "bf16")
    _, sxt = m.mx_quantize_rowwise_tiled(x)
    _, swt = m.mx_quantize_rowwise_tiled(w)
    b = m.mx_grouped_gemm_fwd_tiled(qx, sxt, qw, swt, offs, N, "bf16")
    assert torch.equal(a, b), "full-size fwd: tiled and row-major differ"
    del a, b, qx, sx, qw, sw, sxt, swt
    qdy, sdy = m.mx_quantize_rowwise(dy)
    ldw = m.mx_colwise_ld(G * N)
    qwT, swT = m.mx_quantize_colwise(w, None, ld=ldw)
    a = m.mx_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs, K, "bf16")
    del qwT
    _, sdyt = m.mx_quantize_rowwise_tiled(dy)
    qwTt, swTt = m.mx_quantize_colwise_tiled(w, None, ld=ldw)
    b = m.mx_grouped_gemm_dgrad_tiled(qdy, sdyt, qwTt, swTt, offs, K, "bf16")
    assert torch.equal(a, b), "full-size dgrad: tiled and row-major differ"
    del a, b, qwTt, swTt, qdy, sdy, sdyt
    ld = m.mx_colwise_ld(M, G)
    _, _, qdyT, sdyT = m.mx_quantize_dual(dy, offs, ld=ld)
    _, _, qxT, sxT = m.mx_quantize_dual(x, offs, ld=ld)
    a = m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, M, "f32")
    del qdyT, qxT
    _, _, qdyTt, sdyTt = m.mx_quantize_dual_tiled(dy, offs, ld=ld)
    _, _, qxTt, sxTt = m.mx_quantize_dual_tiled(x, offs, ld=ld)
    b = m.mx_grouped_gemm_wgrad_tiled(qdyTt, sdyTt, qxTt, sxTt, offs, M, "f32")
    assert torch.equal(a, b), "full-size wgrad: tiled and row-major differ"
    del a, b
    torch.cuda.empty_cache()


def test_swiglu_tiled_column_wise_h():
    """The gated forward in the tiled layouts (tiled scales of X and W in, sh, qhT, shT tiled out): Y, qh
    and sh the same bits as the row-major variant (sh permuted); qhT / shT bit-exact against the
    oracle's column-wise quantisation of the kernel's fp32 H, permuted into tiles (experts of 0, 1, 31,
    33, 255, 256, 257 rows; padded ldh)."""
    m = require_gpu()
    rng = np.random.default_rng(85)
    for sizes, N, K in (([0, 1, 31, 33, 255, 0, 256, 257], 256, 256), ([300], 512, 256)):
        offs, x, w, _ = _layer(rng, sizes, N, K)
        M, G = int(offs[-1]), len(sizes)
        H = N // 2
        offs_d = dev(offs)
        qx, sx = m.mx_quantize_rowwise(dev(x))
        qw, sw = m.mx_quantize_rowwise(dev(w))
        _, sxt = m.mx_quantize_rowwise_tiled(dev(x))
        _, swt = m.mx_quantize_rowwise_tiled(dev(w))
        for extra in (0, 128):
            ldh = m.mx_colwise_ld(M, G) + extra
            y0, qh0, sh0, qhT0, shT0 = m.mx_grouped_gemm_fwd_swiglu(qx, sx, qw, sw, offs_d, N, colwise=True, ldh=ldh)
            qhT, shT = _filled((ldh // 128, H, 128)), _filled((ldh // 128, H, 4))
            sh = _filled((H // 128, M, 4))
            y, qh, sh, qhT, shT, h = m.mx_grouped_gemm_fwd_swiglu_tiled(qx, sxt, qw, swt, offs_d, N, sh=sh,
                                                                        with_h=True, qhT=qhT, shT=shT)
            assert torch.equal(y, y0) and torch.equal(qh, qh0)
            same_bytes((host(sh),), (oracle.mx_scales_tiled(host(sh0)),), "sh tiled vs row-major")
            qo, so = oracle.mx_quantize_colwise_values(host(h).astype(np.float64), offs, ldh)
            same_bytes((host(qhT), host(shT)), _tiles(qo, so), f"H tiled {sizes} ldh {ldh}")
            same_bytes((host(qhT), host(shT)), _tiles(host(qhT0), host(shT0)), "H tiled vs row-major")


@pytest.mark.parametrize("fast", [False, True])
def test_tiled_max_expert_count(fast):
    """1024 experts, most of them empty: the tiled dual quantiser bit-exact against the oracle, and the
    three GEMMs on tiled operands give the row-major launches' bits (empty experts' dW zero)."""
    m = require_gpu()
    rng = np.random.default_rng(87)
    G, N, K = 1024, 256, 384
    sizes = np.zeros(G, np.int64)
    busy = rng.choice(G - 1, 50, replace=False)
    sizes[busy] = rng.integers(1, 300, busy.size)
    sizes[G - 1] = 33
    offs, x, w, dy = _layer(rng, sizes, N, K)
    M = int(offs[-1])
    offs_d = dev(offs)
    ld = m.mx_colwise_ld(M, G)
    _dual_tiled_equal(m, x, offs, ld)
    qx, sx, qxT, sxT = m.mx_quantize_dual(dev(x), offs_d, ld=ld)
    qdy, sdy, qdyT, sdyT = m.mx_quantize_dual(dev(dy), offs_d, ld=ld)
    _, sxt, qxTt, sxTt = m.mx_quantize_dual_tiled(dev(x), offs_d, ld=ld)
    _, sdyt, qdyTt, sdyTt = m.mx_quantize_dual_tiled(dev(dy), offs_d, ld=ld)
    qw, sw = m.mx_quantize_rowwise(dev(w))
    _, swt = m.mx_quantize_rowwise_tiled(dev(w))
    ldw = m.mx_colwise_ld(G * N)
    qwT, swT = m.mx_quantize_colwise(dev(w), None, ld=ldw)
    qwTt, swTt = m.mx_quantize_colwise_tiled(dev(w), None, ld=ldw)
    y = m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs_d, N, "f32", fast=fast)
    yt = m.mx_grouped_gemm_fwd_tiled(qx, sxt, qw, swt, offs_d, N, "f32", fast=fast)
    assert torch.equal(y, yt), "fwd: tiled and row-major differ"
    dx = m.mx_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs_d, K, "f32", fast=fast)
    dxt = m.mx_grouped_gemm_dgrad_tiled(qdy, sdyt, qwTt, swTt, offs_d, K, "f32", fast=fast)
    assert torch.equal(dx, dxt), "dgrad: tiled and row-major differ"
    dw = m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs_d, M, "f32", fast=fast)
    dwt = m.mx_grouped_gemm_wgrad_tiled(qdyTt, sdyTt, qxTt, sxTt, offs_d, M, "f32", fast=fast)
    assert torch.equal(dw, dwt), "wgrad: tiled and row-major differ"
    assert not host(dwt)[sizes == 0].any(), "an empty expert's weight gradient is not zero"
