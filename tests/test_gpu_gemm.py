"""GPU parity of the grouped GEMMs against the float64 oracle:
|gpu - ref| <= 1e-5 * sum_k |a_k b_k| per element (bf16 outputs: plus half a bf16 ulp)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_rows, dev, host, random_bf16, require_gpu, same_bytes
from workloads import make_workload, random_offsets, routing_offsets

pytestmark = pytest.mark.gpu


class Layer:
    """Host inputs of one expert layer plus the MX operands the oracle quantises itself."""

    def __init__(self, offs, x, w, dy, N, K):
        self.offs, self.x, self.w, self.dy, self.N, self.K = np.asarray(offs, np.int32), x, w, dy, N, K
        self.G = len(self.offs) - 1
        self.M = int(self.offs[-1])


def _rand_layer(rng, sizes, N, K, w_std=0.05, outliers=0.0):
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    return Layer(offs, random_bf16(rng, (M, K), outlier_frac=outliers), random_bf16(rng, (G * N, K), w_std),
                 random_bf16(rng, (M, N), outlier_frac=outliers), N, K)


# Full-rate FP8 feed: the MFMA truncates each 8-product run to 14 bits below the run's largest product,
# so |err| <= 7 * 2^-13 * sum_runs max|p| + fp32 rounding <= 2^-10 * sum |a b| (derived from the
# measured arithmetic of the instruction; the precise feed meets the 1e-5 bound).
FAST_REL = 2.0 ** -10


def _check(got, ref, bound, dt, what, rel=oracle.gemm.REL_TOL):
    ok, worst, idx = oracle.check_gemm(got, ref, bound, dt, rel=rel)
    assert ok, f"{what}: worst |err|/tol = {worst:.3g} at flat index {idx} (got {got.reshape(-1)[idx]!r}, " \
               f"ref {ref.reshape(-1)[idx]!r}, bound {bound.reshape(-1)[idx]!r})"
    return worst


def _gpu_out(t):
    a = host(t)
    if t.dtype == torch.bfloat16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def run_layer(m, L, dt="f32", rows=None, wgrad_groups=None, n_idx=None, k_idx=None, check=("fwd", "dgrad", "wgrad"),
              fast=False):
    """Quantise on the GPU, run the GEMMs, compare with the oracle evaluated on the GPU's quantised
    operands (copied back).  Those bytes are first compared with the oracle's own quantisation of the
    bf16 inputs: every activation row (column-wise: every n / k row) the sampled outputs read, and a
    sample of the weight rows."""
    offs_d = dev(L.offs)
    x, w, dy = dev(L.x), dev(L.w), dev(L.dy)
    rel = FAST_REL if fast else oracle.gemm.REL_TOL
    r_chk = np.arange(L.M) if rows is None else np.asarray(rows, np.int64)
    worst = {}
    if "fwd" in check:
        qx, sx = m.mx_quantize_rowwise(x)
        qw, sw = m.mx_quantize_rowwise(w)
        y = m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs_d, L.N, dt, fast=fast)
        hq = [host(t) for t in (qx, sx, qw, sw)]
        same_bytes((hq[0][r_chk], hq[1][r_chk]), oracle.mx_quantize_rowwise(L.x[r_chk]), "X row-wise")
        w_chk = check_rows(L.G * L.N, None, 70)
        same_bytes((hq[2][w_chk], hq[3][w_chk]), oracle.mx_quantize_rowwise(L.w[w_chk]), "W row-wise")
        ref, bnd = oracle.mx_gemm_fwd(*hq, L.offs, L.N, rows=rows)
        got = _gpu_out(y)[rows] if rows is not None else _gpu_out(y)
        worst["fwd"] = _check(got, ref, bnd, dt, "fwd", rel)
    if "dgrad" in check:
        qdy, sdy = m.mx_quantize_rowwise(dy)
        # the row pitches the benchmark uses (the recommended ones, >= the minimum)
        ldw = m.mx_colwise_ld(L.G * L.N)
        qwT, swT = m.mx_quantize_colwise(w, None, ld=ldw)
        dx = m.mx_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs_d, L.K, dt, fast=fast)
        hq = [host(t) for t in (qdy, sdy, qwT, swT)]
        same_bytes((hq[0][r_chk], hq[1][r_chk]), oracle.mx_quantize_rowwise(L.dy[r_chk]), "dY row-wise")
        k_chk = check_rows(L.K, None, 71, cap=32)
        same_bytes((hq[2][k_chk], hq[3][k_chk]), oracle.mx_quantize_colwise(L.w[:, k_chk], None, ldw), "W column-wise")
        ref, bnd = oracle.mx_gemm_dgrad(*hq, L.offs, L.N, L.K, rows=rows)
        got = _gpu_out(dx)[rows] if rows is not None else _gpu_out(dx)
        worst["dgrad"] = _check(got, ref, bnd, dt, "dgrad", rel)
    if "wgrad" in check:
        ld = m.mx_colwise_ld(L.M, L.G)
        assert ld >= oracle.mx_colwise_ld_min(L.M, L.G)
        qdyT, sdyT = m.mx_quantize_colwise(dy, offs_d, ld=ld)
        qxT, sxT = m.mx_quantize_colwise(x, offs_d, ld=ld)
        dw = m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs_d, L.M, dt, fast=fast)
        hq = [host(t) for t in (qdyT, sdyT, qxT, sxT)]
        n_chk = np.arange(L.N) if n_idx is None else np.asarray(n_idx)
        k_chk = np.arange(L.K) if k_idx is None else np.asarray(k_idx)
        same_bytes((hq[0][n_chk], hq[1][n_chk]), oracle.mx_quantize_colwise(L.dy[:, n_chk], L.offs, ld), "dY column-wise")
        same_bytes((hq[2][k_chk], hq[3][k_chk]), oracle.mx_quantize_colwise(L.x[:, k_chk], L.offs, ld), "X column-wise")
        ref, bnd = oracle.mx_gemm_wgrad(*hq, L.offs, L.N, L.K, groups=wgrad_groups, n_idx=n_idx, k_idx=k_idx)
        got = _gpu_out(dw)
        if wgrad_groups is not None:
            got = got[np.asarray(wgrad_groups)]
        if n_idx is not None:
            got = got[:, np.asarray(n_idx)]
        if k_idx is not None:
            got = got[:, :, np.asarray(k_idx)]
        worst["wgrad"] = _check(got, ref, bnd, dt, "wgrad", rel)
    return worst


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tiny_workload_all_three(dt):
    m = require_gpu()
    lay = make_workload("tiny").layers[0]
    w = run_layer(m, Layer(lay.offs, lay.x, lay.w.reshape(-1, lay.K), lay.dy, lay.N, lay.K), dt)
    print("worst err/tol", w)


def test_ragged_groups_short_contractions():
    """Short contractions; experts of 0, 1, 17, 33, 129 rows."""
    m = require_gpu()
    rng = np.random.default_rng(30)
    L = _rand_layer(rng, [0, 1, 17, 0, 33, 129, 5], 256, 384, outliers=0.002)
    print(run_layer(m, L))


def test_ragged_groups_long_contractions():
    """Long contractions (K = 2048 forward, N = 1024 dgrad)."""
    m = require_gpu()
    rng = np.random.default_rng(31)
    L = _rand_layer(rng, [3, 0, 130, 257, 64], 1024, 2048)
    print(run_layer(m, L, check=("fwd", "dgrad")))


def test_wgrad_scale_rows_both_paths():
    """The weight gradient reads its scale rows through registers (row pitch not a multiple of 128) or
    straight into LDS as aligned words from the aligned-down block before the expert's first (pitch a
    multiple of 128; the leading blocks are not loaded and must add nothing).  Experts start at blocks
    of every residue mod 4 and end in partial stages, some in the stage they start in; both paths must
    match the oracle."""
    m = require_gpu()
    rng = np.random.default_rng(39)
    # 32-blocks per expert 0, 3, 2, 4, 7, 1, 5, 2, 6, 1, 1, 3: first blocks 0, 0, 3, 5, 9, 16, 17, 22,
    # 24, 30, 31, 32.  The one-block experts at 30 and 31 each fill one stage's block 2 or 3 of 4 at the
    # aligned pitch: the first has leading and trailing blocks outside it, the second leading ones.
    sizes = [0, 70, 40, 128, 200, 5, 150, 33, 180, 20, 32, 90]
    L = _rand_layer(rng, sizes, 256, 384, outliers=0.002)
    offs_d = dev(L.offs)
    x, dy = dev(L.x), dev(L.dy)
    ld_min = oracle.mx_colwise_ld_min(L.M, L.G)
    assert ld_min % 128 != 0
    for ld in (ld_min, m.mxmoe_pitch(ld_min)):
        qdyT, sdyT = m.mx_quantize_colwise(dy, offs_d, ld=ld)
        qxT, sxT = m.mx_quantize_colwise(x, offs_d, ld=ld)
        hq = [host(t) for t in (qdyT, sdyT, qxT, sxT)]
        same_bytes(hq[:2], oracle.mx_quantize_colwise(L.dy, L.offs, ld), f"dY column-wise ld={ld}")
        same_bytes(hq[2:], oracle.mx_quantize_colwise(L.x, L.offs, ld), f"X column-wise ld={ld}")
        ref, bnd = oracle.mx_gemm_wgrad(*hq, L.offs, L.N, L.K)
        for dt in ("f32", "bf16"):
            dw = m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs_d, L.M, dt)
            print("wgrad ld", ld, dt, _check(_gpu_out(dw), ref, bnd, dt, f"wgrad ld={ld} {dt}"))
        # the full-rate FP8 feed (the same two scale paths; its own tolerance)
        dw = m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs_d, L.M, "f32", fast=True)
        print("wgrad fast ld", ld, _check(_gpu_out(dw), ref, bnd, "f32", f"fast wgrad ld={ld}", rel=FAST_REL))


def test_dgrad_padded_weight_pitch():
    """dgrad reads the column-wise weight copy at any row pitch ldw >= G*N: a pitch whose scale rows are
    aligned words (direct-to-LDS scale loads) and one whose are not (register-staged scale words)."""
    m = require_gpu()
    rng = np.random.default_rng(40)
    L = _rand_layer(rng, [0, 5, 130, 1, 300], 256, 384, outliers=0.002)
    offs_d = dev(L.offs)
    qdy, sdy = m.mx_quantize_rowwise(dev(L.dy))
    w = dev(L.w)
    for extra in (384, 32):
        ldw = L.G * L.N + extra
        qwT, swT = m.mx_quantize_colwise(w, None, ld=ldw)
        hq = [host(t) for t in (qdy, sdy, qwT, swT)]
        same_bytes(hq[:2], oracle.mx_quantize_rowwise(L.dy), "dY row-wise")
        same_bytes(hq[2:], oracle.mx_quantize_colwise(L.w, None, ldw), f"W column-wise ldw={ldw}")
        ref, bnd = oracle.mx_gemm_dgrad(*hq, L.offs, L.N, L.K)
        for dt in ("f32", "bf16"):
            dx = m.mx_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs_d, L.K, dt)
            print("dgrad ldw", ldw, dt, _check(_gpu_out(dx), ref, bnd, dt, f"dgrad ldw={ldw} {dt}"))


def test_wgrad_mixed_expert_sizes():
    """Experts of very different sizes in one launch (wgrad contraction length varies per expert)."""
    m = require_gpu()
    rng = np.random.default_rng(32)
    L = _rand_layer(rng, [1500, 0, 17, 1024, 1023, 2100], 256, 256)
    print(run_layer(m, L, check=("wgrad",)))


def test_single_group_and_empty_batch():
    m = require_gpu()
    rng = np.random.default_rng(33)
    print(run_layer(m, _rand_layer(rng, [200], 128, 1024)))
    # M = 0: forward / dgrad are no-ops, wgrad writes zeros
    L = _rand_layer(rng, [0, 0], 128, 256)
    dw = torch.full((2, 128, 256), 7.0, device="cuda")
    ld = oracle.mx_colwise_ld_min(0, 2)
    qT = torch.zeros((128, ld), dtype=torch.uint8, device="cuda")
    sT = torch.zeros((128, ld // 32), dtype=torch.uint8, device="cuda")
    qX = torch.zeros((256, ld), dtype=torch.uint8, device="cuda")
    sX = torch.zeros((256, ld // 32), dtype=torch.uint8, device="cuda")
    m.mx_grouped_gemm_wgrad(qT, sT, qX, sX, dev(L.offs), 0, "f32", dw=dw)
    torch.cuda.synchronize()
    assert not dw.any()


def test_determinism_and_no_out_of_bounds_writes():
    m = require_gpu()
    rng = np.random.default_rng(34)
    L = _rand_layer(rng, [7, 300, 0, 45], 256, 1024)
    offs = dev(L.offs)
    qx, sx = m.mx_quantize_rowwise(dev(L.x))
    qw, sw = m.mx_quantize_rowwise(dev(L.w))
    guard = 4096
    buf = torch.full((L.M * L.N + 2 * guard,), -3.0, device="cuda")
    y = buf[guard:guard + L.M * L.N].view(L.M, L.N)
    m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs, L.N, y=y)
    y1 = y.clone()
    m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs, L.N, y=y)
    torch.cuda.synchronize()
    assert torch.equal(y, y1)
    assert torch.all(buf[:guard] == -3.0) and torch.all(buf[guard + L.M * L.N:] == -3.0)


@pytest.mark.parametrize("fast", [False, True])
def test_tiny_and_ragged_fast_feed(fast):
    """The full-rate FP8 feed within its derived bound (and the precise feed within 1e-5)."""
    m = require_gpu()
    lay = make_workload("tiny").layers[0]
    print(run_layer(m, Layer(lay.offs, lay.x, lay.w.reshape(-1, lay.K), lay.dy, lay.N, lay.K), fast=fast))
    rng = np.random.default_rng(38)
    print(run_layer(m, _rand_layer(rng, [0, 1, 17, 300, 1100], 256, 1024, outliers=0.002), fast=fast))


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("name", ["dsv3_16b", "dsv3_671b_shard", "llama4_scout"])
def test_full_size_sampled(name, fast):
    """Full-size layers in the launch configuration the benchmark times; the oracle checks sampled
    rows (forward, dgrad) and sampled (expert, n, k) entries (wgrad), every expert included.  The
    full-rate FP8 feed against its own bound."""
    m = require_gpu()
    wl = make_workload(name)
    rng = np.random.default_rng(35)
    for lay in wl.layers:
        offs = lay.offs.astype(np.int64)
        rows = []
        for g in range(lay.G):
            if offs[g + 1] > offs[g]:
                rows += [offs[g], offs[g + 1] - 1] + list(rng.integers(offs[g], offs[g + 1], size=6))
        rows = np.unique(np.array(rows, np.int64))
        L = Layer(lay.offs, lay.x, lay.w.reshape(-1, lay.K), lay.dy, lay.N, lay.K)
        n_idx = np.unique(np.concatenate([[0, lay.N - 1], rng.choice(lay.N, 24, replace=False)]))
        k_idx = np.unique(np.concatenate([[0, lay.K - 1], rng.choice(lay.K, 24, replace=False)]))
        w = run_layer(m, L, "bf16" if lay.name == "gate_up" else "f32", rows=rows, n_idx=n_idx, k_idx=k_idx,
                      fast=fast)
        print(name, lay.name, "fast" if fast else "precise", w)
        torch.cuda.empty_cache()


def test_blockwise_gemms():
    m = require_gpu()
    rng = np.random.default_rng(36)
    for sizes, N, K in (([0, 5, 130, 1, 60], 256, 1024), ([40, 0, 200], 1024, 256)):
        L = _rand_layer(rng, sizes, N, K, w_std=0.02, outliers=0.001)
        offs = dev(L.offs)
        qx, sx = m.fp8bw_quantize_act_1x128(dev(L.x))
        qw, sw, qwT = m.fp8bw_quantize_weight_128x128(dev(L.w), transposed=True)
        same_bytes((host(qx), host(sx)), oracle.bw_quantize_act_1x128(L.x), "bw X 1x128")
        wq = oracle.bw_quantize_weight_128x128(L.w)
        same_bytes((host(qw), host(sw), host(qwT)), (wq[0], wq[1], wq[0].T), "bw W 128x128")
        y = m.fp8bw_grouped_gemm_fwd(qx, sx, qw, sw, offs, N)
        ref, bnd = oracle.bw_gemm_fwd(host(qx), host(sx), host(qw), host(sw), L.offs, N)
        print("bw fwd", _check(_gpu_out(y), ref, bnd, "f32", "bw fwd"))
        qd, sd = m.fp8bw_quantize_act_1x128(dev(L.dy))
        same_bytes((host(qd), host(sd)), oracle.bw_quantize_act_1x128(L.dy), "bw dY 1x128")
        dx = m.fp8bw_grouped_gemm_dgrad(qd, sd, qwT, sw, offs, K)
        ref, bnd = oracle.bw_gemm_dgrad(host(qd), host(sd), host(qw), host(sw), L.offs, N, K)
        print("bw dgrad", _check(_gpu_out(dx), ref, bnd, "f32", "bw dgrad"))


def test_blockwise_fp8_feed():
    """The blockwise GEMMs on the full-rate FP8 feed (each slice's partial from the block-scaled MFMA
    with unit scales, then promoted) against the oracle within that feed's bound; ragged experts."""
    m = require_gpu()
    rng = np.random.default_rng(48)
    L = _rand_layer(rng, [0, 5, 130, 1, 300], 256, 384, w_std=0.02, outliers=0.001)
    offs = dev(L.offs)
    qx, sx = m.fp8bw_quantize_act_1x128(dev(L.x))
    qw, sw, qwT = m.fp8bw_quantize_weight_128x128(dev(L.w), transposed=True)
    same_bytes((host(qx), host(sx)), oracle.bw_quantize_act_1x128(L.x), "bw X 1x128")
    wq = oracle.bw_quantize_weight_128x128(L.w)
    same_bytes((host(qw), host(sw), host(qwT)), (wq[0], wq[1], wq[0].T), "bw W 128x128")
    y = m.fp8bw_grouped_gemm_fwd(qx, sx, qw, sw, offs, L.N, fast=True)
    ref, bnd = oracle.bw_gemm_fwd(host(qx), host(sx), host(qw), host(sw), L.offs, L.N)
    print("bw fast fwd", _check(_gpu_out(y), ref, bnd, "f32", "bw fast fwd", rel=FAST_REL))
    qd, sd = m.fp8bw_quantize_act_1x128(dev(L.dy))
    same_bytes((host(qd), host(sd)), oracle.bw_quantize_act_1x128(L.dy), "bw dY 1x128")
    dx = m.fp8bw_grouped_gemm_dgrad(qd, sd, qwT, sw, offs, L.K, fast=True)
    ref, bnd = oracle.bw_gemm_dgrad(host(qd), host(sd), host(qw), host(sw), L.offs, L.N, L.K)
    print("bw fast dgrad", _check(_gpu_out(dx), ref, bnd, "f32", "bw fast dgrad", rel=FAST_REL))
    ld = oracle.bw_colwise_ld_min(L.M, L.G)
    qdT, sdT = m.fp8bw_quantize_colwise_128(dev(L.dy), offs, ld=ld)
    qxT, sxT = m.fp8bw_quantize_colwise_128(dev(L.x), offs, ld=ld)
    same_bytes((host(qdT), host(sdT)), oracle.bw_quantize_colwise_128(L.dy, L.offs, ld), "bw dY 128-token")
    same_bytes((host(qxT), host(sxT)), oracle.bw_quantize_colwise_128(L.x, L.offs, ld), "bw X 128-token")
    dw = m.fp8bw_grouped_gemm_wgrad(qdT, sdT, qxT, sxT, offs, L.M, "f32", fast=True)
    ref, bnd = oracle.bw_gemm_wgrad(host(qdT), host(sdT), host(qxT), host(sxT), L.offs, L.N, L.K)
    print("bw fast wgrad", _check(_gpu_out(dw), ref, bnd, "f32", "bw fast wgrad", rel=FAST_REL))


@pytest.mark.parametrize("pow2", [False, True])
def test_blockwise_full_size_sampled(pow2):
    """The blockwise recipe on the DeepSeek-V3-16B layer tensors (sampled rows); with power-of-two
    scales through the _pow2 GEMMs (the MX kernel), whose weight gradient is also sampled (two experts,
    sampled n and k)."""
    m = require_gpu()
    wl = make_workload("dsv3_16b_blockwise")
    rng = np.random.default_rng(37)
    fwd = m.fp8bw_grouped_gemm_fwd_pow2 if pow2 else m.fp8bw_grouped_gemm_fwd
    dgrad = m.fp8bw_grouped_gemm_dgrad_pow2 if pow2 else m.fp8bw_grouped_gemm_dgrad
    for lay in wl.layers:
        offs_d = dev(lay.offs)
        rows = np.unique(rng.choice(lay.M, 64, replace=False))
        qx, sx = m.fp8bw_quantize_act_1x128(dev(lay.x), pow2=pow2)
        w2 = lay.w.reshape(-1, lay.K)
        qw, sw, qwT = m.fp8bw_quantize_weight_128x128(dev(w2), transposed=True, pow2=pow2)
        y = fwd(qx, sx, qw, sw, offs_d, lay.N)
        hqw, hsw = host(qw), host(sw)
        same_bytes((host(qx)[rows], host(sx)[rows]), oracle.bw_quantize_act_1x128(lay.x[rows], pow2=pow2), "bw X 1x128")
        hqwT = host(qwT)
        for band in rng.choice(w2.shape[0] // 128, 4, replace=False):       # sampled 128-row weight bands
            r = slice(128 * band, 128 * band + 128)
            wq = oracle.bw_quantize_weight_128x128(w2[r], pow2=pow2)
            same_bytes((hqw[r], hsw[band:band + 1], hqwT[:, r]), (wq[0], wq[1], wq[0].T), "bw W 128x128")
        ref, bnd = oracle.bw_gemm_fwd(host(qx), host(sx), hqw, hsw, lay.offs, lay.N, rows=rows)
        print(lay.name, "bw fwd", _check(_gpu_out(y)[rows], ref, bnd, "f32", "bw fwd"))
        qd, sd = m.fp8bw_quantize_act_1x128(dev(lay.dy), pow2=pow2)
        same_bytes((host(qd)[rows], host(sd)[rows]), oracle.bw_quantize_act_1x128(lay.dy[rows], pow2=pow2), "bw dY 1x128")
        dx = dgrad(qd, sd, qwT, sw, offs_d, lay.K)
        ref, bnd = oracle.bw_gemm_dgrad(host(qd), host(sd), hqw, hsw, lay.offs, lay.N, lay.K, rows=rows)
        print(lay.name, "bw dgrad", _check(_gpu_out(dx)[rows], ref, bnd, "f32", "bw dgrad"))
        if pow2:
            ld = m.fp8bw_colwise_ld_min(lay.M, lay.G)
            qdT, sdT = m.fp8bw_quantize_colwise_128(dev(lay.dy), offs_d, ld=ld, pow2=True)
            qxT, sxT = m.fp8bw_quantize_colwise_128(dev(lay.x), offs_d, ld=ld, pow2=True)
            dw = m.fp8bw_grouped_gemm_wgrad_pow2(qdT, sdT, qxT, sxT, offs_d, lay.M, "f32")
            sizes = np.diff(lay.offs.astype(np.int64))
            groups = [int(np.argmax(sizes)), int(rng.choice(np.flatnonzero(sizes > 0)))]
            n_idx = np.sort(rng.choice(lay.N, 24, replace=False))
            k_idx = np.sort(rng.choice(lay.K, 24, replace=False))
            hd = (host(qdT), host(sdT), host(qxT), host(sxT))
            same_bytes((hd[0][n_idx], hd[1][n_idx]), oracle.bw_quantize_colwise_128(lay.dy[:, n_idx], lay.offs, ld, pow2=True),
                       "bw dY 128-token")
            same_bytes((hd[2][k_idx], hd[3][k_idx]), oracle.bw_quantize_colwise_128(lay.x[:, k_idx], lay.offs, ld, pow2=True),
                       "bw X 128-token")
            ref, bnd = oracle.bw_gemm_wgrad(*hd, lay.offs, lay.N, lay.K, groups=groups, n_idx=n_idx, k_idx=k_idx)
            got = _gpu_out(dw)[np.asarray(groups)][:, n_idx][:, :, k_idx]
            print(lay.name, "bw wgrad", _check(got, ref, bnd, "f32", "bw wgrad"))
        torch.cuda.empty_cache()


def test_precise_feed_keeps_small_products_of_a_run():
    """A product 2^17 times smaller than the largest one of its 8-element contraction run is summed
    exactly by the precise feed (the block-scaled FP8 MFMA keeps only about 14 bits below the run's
    largest product).  The sums are exact in fp32, so the result must equal the oracle bit for bit."""
    m = require_gpu()
    K, N = 128, 256
    offs = np.array([0, 1], np.int32)
    qw = np.full((N, K), 0x38, np.uint8)                 # 1.0
    sw = np.full((N, K // 32), 127, np.uint8)
    cases = []
    for j in (1, 3, 7, 8, 40, 127):
        qx = np.zeros((1, K), np.uint8)
        qx[0, 0], qx[0, j] = 0x78, 0x01                  # 256 and 2^-9
        cases.append(qx)
    qx = np.zeros((1, K), np.uint8)
    qx[0, 0], qx[0, 1:8] = 0x78, 0x1F                    # 256 and seven times 0.1171875
    cases.append(qx)
    sx = np.full((1, K // 32), 127, np.uint8)
    for qx in cases:
        y = m.mx_grouped_gemm_fwd(dev(qx), dev(sx), dev(qw), dev(sw), dev(offs), N, "f32")
        ref, _ = oracle.mx_gemm_fwd(qx, sx, qw, sw, offs, N)
        assert np.array_equal(_gpu_out(y), ref), (np.flatnonzero(qx[0]), _gpu_out(y)[0, 0], ref[0, 0])


def test_fp8_feed_truncates_each_run_of_eight():
    """The full-rate FP8 feed's arithmetic, pinned through the C-ABI (X row against W = 1, unit scales):
    a product 2^-9 beside 256 in the same run of 8 contraction elements (positions 1..7) is dropped,
    and kept in every other run (positions 8..127, across 32-blocks and MFMA k-steps); seven products
    0.1171875 beside 256 in one run add 7 * 0.09375 (each truncated toward zero to a multiple of
    2^(8 - 13)), and their negatives subtract as much; a run without a large product is exact."""
    m = require_gpu()
    K, N = 128, 256
    offs = np.array([0, 1], np.int32)
    qw = np.full((N, K), 0x38, np.uint8)                 # 1.0
    sw = np.full((N, K // 32), 127, np.uint8)
    sx = np.full((1, K // 32), 127, np.uint8)
    cases = []
    for j in range(1, K):
        qx = np.zeros((1, K), np.uint8)
        qx[0, 0], qx[0, j] = 0x78, 0x01                  # 256 and 2^-9
        cases.append((qx, 256.0 if j < 8 else 256.0 + 2.0 ** -9))
    for big, sign, want in ((0, 0x00, 256.0 + 7 * 0.09375), (0, 0x80, 256.0 - 7 * 0.09375),
                            (72, 0x00, 256.0 + 7 * 0.09375)):
        qx = np.zeros((1, K), np.uint8)
        qx[0, big], qx[0, big + 1:big + 8] = 0x78, 0x1F | sign       # 256 and seven times +-0.1171875
        cases.append((qx, want))
    qx = np.zeros((1, K), np.uint8)
    qx[0, 16:24] = 0x1F                                   # a run of small products only: exact
    qx[0, 0] = 0x78
    cases.append((qx, 256.0 + 8 * 0.1171875))
    X = np.concatenate([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    offs = np.array([0, len(cases)], np.int32)
    sxs = np.repeat(sx, len(cases), axis=0)
    y = m.mx_grouped_gemm_fwd(dev(X), dev(sxs), dev(qw), dev(sw), dev(offs), N, "f32", fast=True)
    got = _gpu_out(y)
    assert np.all(got == got[:, :1]), "every output column sees the same products"
    bad = np.flatnonzero(got[:, 0] != want)
    assert bad.size == 0, [(int(i), got[i, 0], want[i]) for i in bad[:6]]
    # the precise feed sums the same rows exactly
    y = m.mx_grouped_gemm_fwd(dev(X), dev(sxs), dev(qw), dev(sw), dev(offs), N, "f32")
    ref, _ = oracle.mx_gemm_fwd(X, sxs, qw, sw, offs, N)
    assert np.array_equal(_gpu_out(y), ref)


def _block_scaled_bf16(rng, shape, block_axis, span=40):
    """N(0,1) values whose 32-element blocks along `block_axis` are each scaled by 2^u, u ~ U{-span..span}."""
    from workloads import f32_to_bf16_bits
    x = rng.standard_normal(shape).astype(np.float32)
    if block_axis == 1:
        u = rng.integers(-span, span + 1, size=(shape[0], shape[1] // 32))
        x *= np.repeat(np.exp2(u), 32, axis=1).astype(np.float32)
    else:
        u = rng.integers(-span, span + 1, size=(-(-shape[0] // 32), shape[1]))
        x *= np.repeat(np.exp2(u), 32, axis=0)[:shape[0]].astype(np.float32)
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("fast", [False, True])
def test_per_block_scales_over_a_wide_range(fast):
    """Every 32-block carries its own scale (2^-40 .. 2^40 relative): a scale paired with the wrong
    block would miss the oracle by orders of magnitude.  Blocks vary along the contraction axis of
    each GEMM (row-wise copies along K / N, column-wise copies down the token rows)."""
    m = require_gpu()
    rng = np.random.default_rng(40)
    sizes, N, K = [33, 0, 290, 5, 64], 256, 512
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    L = Layer(offs, _block_scaled_bf16(rng, (M, K), 1), _block_scaled_bf16(rng, (G * N, K), 1),
              _block_scaled_bf16(rng, (M, N), 1), N, K)
    print(run_layer(m, L, check=("fwd",), fast=fast))
    L = Layer(offs, _block_scaled_bf16(rng, (M, K), 0), _block_scaled_bf16(rng, (G * N, K), 0),
              _block_scaled_bf16(rng, (M, N), 0), N, K)
    print(run_layer(m, L, check=("dgrad", "wgrad"), fast=fast))


def _bw_wgrad_case(m, L, dt, groups=None, n_idx=None, k_idx=None):
    ld = oracle.bw_colwise_ld_min(L.M, L.G)
    offs = dev(L.offs)
    qd, sd = m.fp8bw_quantize_colwise_128(dev(L.dy), offs, ld=ld)
    qx, sx = m.fp8bw_quantize_colwise_128(dev(L.x), offs, ld=ld)
    dw = m.fp8bw_grouped_gemm_wgrad(qd, sd, qx, sx, offs, L.M, dt)
    n_chk = check_rows(L.N, n_idx)
    k_chk = check_rows(L.K, k_idx)
    same_bytes((host(qd)[n_chk], host(sd)[n_chk]), oracle.bw_quantize_colwise_128(L.dy[:, n_chk], L.offs, ld), "bw dY 128-token")
    same_bytes((host(qx)[k_chk], host(sx)[k_chk]), oracle.bw_quantize_colwise_128(L.x[:, k_chk], L.offs, ld), "bw X 128-token")
    ref, bnd = oracle.bw_gemm_wgrad(host(qd), host(sd), host(qx), host(sx), L.offs, L.N, L.K,
                                    groups=groups, n_idx=n_idx, k_idx=k_idx)
    got = _gpu_out(dw)
    if groups is not None:
        got = got[np.ix_(groups, n_idx, k_idx)]
    return _check(got, ref, bnd, dt, f"bw wgrad {dt}")


def test_blockwise_wgrad():
    """Blockwise wgrad (128-token blocks promoted with the dY and X row scales) on ragged experts,
    including empty ones (zero gradient written), fp32 and bf16 outputs."""
    m = require_gpu()
    rng = np.random.default_rng(38)
    for sizes, N, K in (([0, 5, 130, 1, 300], 256, 384), ([129, 0, 0, 17], 128, 256)):
        L = _rand_layer(rng, sizes, N, K, outliers=0.001)
        for dt in ("f32", "bf16"):
            print("bw wgrad", sizes, dt, _bw_wgrad_case(m, L, dt))
    # no routed rows at all: every dW_g is written as zero
    ld = oracle.bw_colwise_ld_min(0, 2)
    offs = dev(np.zeros(3, np.int32))
    qd, sd = m.fp8bw_quantize_colwise_128(dev(np.zeros((1, 128), np.uint16))[:0], offs, ld=ld)
    dw = m.fp8bw_grouped_gemm_wgrad(qd, sd, qd, sd, offs, 0, "f32", dw=torch.full((2, 128, 128), 7.0, device="cuda"))
    assert not host(dw).any()


def test_blockwise_wgrad_full_size_sampled():
    """DeepSeek-V3-16B layer tensors (64 experts): the full launches, sampled experts and n / k."""
    m = require_gpu()
    wl = make_workload("dsv3_16b_blockwise")
    rng = np.random.default_rng(39)
    for lay in wl.layers:
        groups = np.unique(np.concatenate([[0, lay.G - 1], rng.choice(lay.G, 4, replace=False)]))
        n_idx = np.unique(np.concatenate([[0, lay.N - 1], rng.choice(lay.N, 24, replace=False)]))
        k_idx = np.unique(np.concatenate([[0, lay.K - 1], rng.choice(lay.K, 24, replace=False)]))
        print(lay.name, "bw wgrad", _bw_wgrad_case(m, lay, "f32", groups, n_idx, k_idx))
        torch.cuda.empty_cache()


def _swiglu_case(m, L, rows=None, ldh_extra=0, u_idx=None):
    """Fused gate+up forward: Y against the oracle forward; the kernel's fp32 H against fp64 SwiGLU of
    the oracle's Y within the propagated GEMM bound; qh / sh (row-wise) and qhT / shT (column-wise,
    written into buffers pre-filled with 0xAB so that pads and the tail must be written) bit-exact
    against the oracle's MX quantisation of that same fp32 H (u_idx: the sampled hidden units whose
    column-wise rows are compared)."""
    offs = dev(L.offs)
    qx, sx = m.mx_quantize_rowwise(dev(L.x))
    qw, sw = m.mx_quantize_rowwise(dev(L.w))
    H = L.N // 2
    ldh = m.mx_colwise_ld(L.M, L.G) + ldh_extra
    qhT = torch.full((H, ldh), 0xAB, dtype=torch.uint8, device="cuda")
    shT = torch.full((H, ldh // 32), 0xAB, dtype=torch.uint8, device="cuda")
    y, qh, sh, qhT, shT, h = m.mx_grouped_gemm_fwd_swiglu(qx, sx, qw, sw, offs, L.N, with_h=True, qhT=qhT, shT=shT)
    hk = host(h).astype(np.float64)
    u_chk = np.arange(H) if u_idx is None else np.asarray(u_idx)
    same_bytes((host(qhT)[u_chk], host(shT)[u_chk]), oracle.mx_quantize_colwise_values(hk[:, u_chk], L.offs, ldh),
               "H column-wise")
    hq = [host(t) for t in (qx, sx, qw, sw)]
    r_chk = np.arange(L.M) if rows is None else np.asarray(rows, np.int64)
    same_bytes((hq[0][r_chk], hq[1][r_chk]), oracle.mx_quantize_rowwise(L.x[r_chk]), "X row-wise")
    w_chk = check_rows(L.G * L.N, None, 72)
    same_bytes((hq[2][w_chk], hq[3][w_chk]), oracle.mx_quantize_rowwise(L.w[w_chk]), "W row-wise")
    ref, bnd = oracle.mx_gemm_fwd(*hq, L.offs, L.N, rows=rows)
    sel = slice(None) if rows is None else rows
    worst_y = _check(_gpu_out(y)[sel], ref, bnd, "bf16", "swiglu y")
    hg = host(h)[sel].astype(np.float64)
    g, u = ref[:, :H], ref[:, H:]
    tol_g = oracle.gemm.REL_TOL * bnd[:, :H] + 2.0 ** -24 * np.abs(g)
    tol_u = oracle.gemm.REL_TOL * bnd[:, H:] + 2.0 ** -24 * np.abs(u)
    href = oracle.swiglu(g, u)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    tol_h = 1.1 * tol_g * np.abs(u) + np.abs(silu) * tol_u + 4e-6 * np.abs(href) + 1e-30
    err = np.abs(hg - href)
    assert np.all(err <= tol_h), f"H: worst err/tol {np.max(err / tol_h):.3g}"
    qo, so = oracle.mx_quantize_rowwise_values(hg)
    assert np.array_equal(host(sh)[sel], so), "H scales differ from the oracle's quantisation of the kernel's H"
    bad = np.argwhere(host(qh)[sel] != qo)
    assert bad.size == 0, f"H codes differ at {bad[:5]}"
    return worst_y, float(np.max(err / tol_h))


def test_swiglu_fused_forward_colwise_edges():
    """Column-wise H from the epilogue: experts of 0, 1, 31, 32, 33, 255, 256 and 257 rows (blocks
    short, whole, and spanning two row tiles), a padded leading dimension, and one expert only."""
    m = require_gpu()
    rng = np.random.default_rng(47)
    L = _rand_layer(rng, [0, 1, 31, 32, 33, 255, 0, 256, 257], 256, 256, w_std=0.05, outliers=0.001)
    print("swiglu colwise", _swiglu_case(m, L, ldh_extra=96))
    L = _rand_layer(rng, [300], 512, 256, w_std=0.05, outliers=0.001)
    print("swiglu colwise one expert", _swiglu_case(m, L))


def test_swiglu_fused_forward():
    m = require_gpu()
    rng = np.random.default_rng(45)
    for sizes, N, K in (([0, 5, 130, 1, 300], 512, 256), ([257, 0, 17], 256, 384)):
        L = _rand_layer(rng, sizes, N, K, w_std=0.05, outliers=0.001)
        print("swiglu", sizes, _swiglu_case(m, L))


def test_swiglu_fused_forward_full_size_sampled():
    """DeepSeek-V3-671B shard gate+up (N = 2H = 4096, K = 7168), sampled rows."""
    m = require_gpu()
    lay = make_workload("dsv3_671b_shard", layers=["gate_up"]).layers[0]
    rng = np.random.default_rng(46)
    rows = np.unique(np.concatenate([[0, lay.M - 1], rng.choice(lay.M, 48, replace=False)]))
    L = Layer(lay.offs, lay.x, lay.w.reshape(-1, lay.K), lay.dy, lay.N, lay.K)
    u_idx = np.unique(np.concatenate([[0, lay.N // 2 - 1], rng.choice(lay.N // 2, 14, replace=False)]))
    print("swiglu full", _swiglu_case(m, L, rows=rows, u_idx=u_idx))
    torch.cuda.empty_cache()
