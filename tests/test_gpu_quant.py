"""GPU parity of the quantisers against the oracle: bit-exact bytes and scales."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, random_bf16, require_gpu
from workloads import f32_to_bf16_bits, make_workload, random_offsets, routing_offsets

pytestmark = pytest.mark.gpu


def _finite_bf16_patterns():
    b = np.arange(65536, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def _rowwise_equal(m, x):
    q, s = m.mx_quantize_rowwise(dev(x))
    qo, so = oracle.mx_quantize_rowwise(x)
    qg, sg = host(q), host(s)
    bad = np.argwhere(qg != qo)
    assert np.array_equal(sg, so), f"scale mismatch at {np.argwhere(sg != so)[:5]}"
    assert bad.size == 0, f"q mismatch at {bad[:5]}: gpu {qg[tuple(bad[0])]:#x} oracle {qo[tuple(bad[0])]:#x}"


def test_rowwise_exhaustive_bf16_as_block_max():
    m = require_gpu()
    p = _finite_bf16_patterns()
    x = np.zeros((len(p), 32), np.uint16)
    x[:, 0] = p
    x[:, 1] = p ^ 0x8000          # the same magnitude with the other sign
    _rowwise_equal(m, x)


@pytest.mark.parametrize("amax", [1.0, 3.0, 2.0 ** -100, 2.0 ** 60, 2.0 ** -121, 448.0 * 2 ** 20])
def test_rowwise_exhaustive_bf16_below_amax(amax):
    m = require_gpu()
    p = _finite_bf16_patterns()
    v = (p.astype(np.uint32) << 16).view(np.float32)
    p = p[np.abs(v) <= amax]
    n = (len(p) + 30) // 31
    x = np.zeros((n, 32), np.uint16)
    flat = np.zeros(n * 31, np.uint16)
    flat[:len(p)] = p
    x[:, :31] = flat.reshape(n, 31)
    x[:, 31] = f32_to_bf16_bits(np.array([amax], np.float32))[0]
    _rowwise_equal(m, x)


def test_rowwise_random_shapes_and_outliers():
    m = require_gpu()
    rng = np.random.default_rng(20)
    for R, C in ((1, 32), (3, 96), (257, 512), (1000, 2048)):
        _rowwise_equal(m, random_bf16(rng, (R, C), outlier_frac=0.01, outlier_mult=1000.0))
    _rowwise_equal(m, random_bf16(rng, (300, 256), std=2.0 ** -125))      # tiny and clamped exponents
    _rowwise_equal(m, random_bf16(rng, (300, 256), std=2.0 ** 100))


def test_rowwise_tiny_workload_tensors():
    m = require_gpu()
    lay = make_workload("tiny").layers[0]
    for t in (lay.x, lay.w.reshape(-1, lay.K), lay.dy):
        _rowwise_equal(m, t)


def _colwise_equal(m, x, offs, ld=None):
    R, C = x.shape
    if offs is None:
        ld = ld or 32 * ((R + 31) // 32)
        qT, sT = m.mx_quantize_colwise(dev(x), None, ld=ld)
    else:
        ld = ld or oracle.mx_colwise_ld_min(R, len(offs) - 1)
        qT, sT = m.mx_quantize_colwise(dev(x), dev(np.asarray(offs, np.int32)), ld=ld)
    qo, so = oracle.mx_quantize_colwise(x, offs, ld)
    qg, sg = host(qT), host(sT)
    assert np.array_equal(sg, so), f"scale mismatch at {np.argwhere(sg != so)[:5]}"
    bad = np.argwhere(qg != qo)
    assert bad.size == 0, f"q mismatch at {bad[:5]}"


def test_colwise_ragged_groups():
    m = require_gpu()
    rng = np.random.default_rng(21)
    for sizes, C in (([17, 0, 33, 1, 70], 64), ([0, 0, 5], 32), ([128], 96), ([31, 32, 33, 0, 64, 1], 160)):
        offs = routing_offsets(sizes)
        _colwise_equal(m, random_bf16(rng, (int(offs[-1]), C), outlier_frac=0.02), offs)
    # larger ld than needed: the extra tail must be zero
    offs = routing_offsets([40, 3])
    _colwise_equal(m, random_bf16(rng, (43, 64)), offs, ld=512)
    # many groups, random sizes with empties
    offs = random_offsets(rng, 3000, 37)
    _colwise_equal(m, random_bf16(rng, (3000, 128), outlier_frac=0.001), offs)


def test_colwise_single_group_weight_layout():
    m = require_gpu()
    rng = np.random.default_rng(22)
    w = random_bf16(rng, (4 * 512, 256), std=0.02)
    _colwise_equal(m, w, None)
    _colwise_equal(m, w, routing_offsets([512] * 4), ld=4 * 512 + 128)


def test_colwise_tiny_workload():
    m = require_gpu()
    lay = make_workload("tiny").layers[0]
    _colwise_equal(m, lay.x, lay.offs)
    _colwise_equal(m, lay.dy, lay.offs)
    _colwise_equal(m, lay.w.reshape(-1, lay.K), None)


def test_blockwise_quantisers():
    m = require_gpu()
    rng = np.random.default_rng(23)
    for R, C in ((1, 128), (37, 384), (300, 1024)):
        x = random_bf16(rng, (R, C), outlier_frac=0.01)
        x[0, :128] = 0                       # an all-zero tile -> scale 1
        q, s = m.fp8bw_quantize_act_1x128(dev(x))
        qo, so = oracle.bw_quantize_act_1x128(x)
        assert np.array_equal(host(s), so)
        assert np.array_equal(host(q), qo)
    for R, C in ((128, 128), (512, 384)):
        w = random_bf16(rng, (R, C), std=0.02, outlier_frac=0.001)
        q, s = m.fp8bw_quantize_weight_128x128(dev(w))
        qo, so = oracle.bw_quantize_weight_128x128(w)
        assert np.array_equal(host(s), so)
        assert np.array_equal(host(q), qo)
        # with the transposed copy: same codes and scales, plus qT == q^T
        q2, s2, qT = m.fp8bw_quantize_weight_128x128(dev(w), transposed=True)
        assert np.array_equal(host(s2), so) and np.array_equal(host(q2), qo)
        assert np.array_equal(host(qT), qo.T)


def test_quantisers_full_size_sampled():
    """DeepSeek-V3-671B shard, gate+up X [65536, 7168] and W: full-size launches, sampled rows/columns."""
    m = require_gpu()
    wl = make_workload("dsv3_671b_shard", layers=["gate_up"])
    lay = wl.layers[0]
    rng = np.random.default_rng(24)
    x = dev(lay.x)
    q, s = m.mx_quantize_rowwise(x)
    rows = np.concatenate([[0, lay.M - 1], rng.choice(lay.M, 300, replace=False)])
    qo, so = oracle.mx_quantize_rowwise(lay.x[rows])
    assert np.array_equal(host(q[rows]), qo) and np.array_equal(host(s[rows]), so)
    cols = np.concatenate([[0, lay.K - 1], rng.choice(lay.K, 40, replace=False)])
    # the minimum row pitch and the recommended one the benchmark uses
    ld_min = oracle.mx_colwise_ld_min(lay.M, lay.G)
    for ld in (ld_min, m.mx_colwise_ld(lay.M, lay.G)):
        qT, sT = m.mx_quantize_colwise(x, dev(lay.offs), ld=ld)
        qo, so = oracle.mx_quantize_colwise(np.ascontiguousarray(lay.x[:, cols]), lay.offs, ld)
        assert np.array_equal(host(qT[cols]), qo) and np.array_equal(host(sT[cols]), so)
        del qT, sT


def _dual_equal(m, x, offs, ld, row_idx=None):
    """Fused dual-layout quantiser against the oracle: all four outputs byte for byte."""
    out = m.mx_quantize_dual(dev(x), None if offs is None else dev(offs), ld=ld,
                             row_idx=None if row_idx is None else dev(row_idx))
    ref = oracle.mx_quantize_dual(x, offs, ld, row_idx)
    for name, g, r in zip(("q", "s", "qT", "sT"), out, ref):
        g = host(g)
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"{name} mismatch at {bad[:5]}"


def test_dual_ragged_groups_and_partial_windows():
    m = require_gpu()
    rng = np.random.default_rng(25)
    sizes = [0, 5, 130, 1, 60, 33, 0]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offs[-1])
    for C in (32, 96, 288, 512, 1056):
        x = random_bf16(rng, (M, C), outlier_frac=0.01, outlier_mult=1000.0)
        ld = oracle.mx_colwise_ld_min(M, len(sizes))
        _dual_equal(m, x, offs, ld)
        _dual_equal(m, x, offs, ld + 96)          # extra tail columns stay zero


def test_dual_single_group_weight_layout():
    m = require_gpu()
    rng = np.random.default_rng(26)
    for R, C in ((4 * 64, 320), (3 * 128, 2048), (37, 64)):
        x = random_bf16(rng, (R, C), std=0.02, outlier_frac=0.001)
        ld = 32 * ((R + 31) // 32)
        _dual_equal(m, x, None, ld)
        _dual_equal(m, x, None, ld + 32)


def test_dual_gather_top2_routing():
    """Routed rows gathered by index (each token twice, in expert order), including two invalid
    indices that the library clamps into range."""
    m = require_gpu()
    rng = np.random.default_rng(27)
    T, C, G = 300, 384, 5
    x = random_bf16(rng, (T, C), outlier_frac=0.01, outlier_mult=100.0)
    experts = np.stack([rng.choice(G, 2, replace=False) for _ in range(T)])    # top-2, distinct
    tok = np.repeat(np.arange(T), 2)
    exp = experts.reshape(-1)
    order = np.argsort(exp, kind="stable")
    row_idx = tok[order].astype(np.int32)
    row_idx[7] = -3
    row_idx[11] = T + 40
    sizes = np.bincount(exp, minlength=G)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    ld = oracle.mx_colwise_ld_min(2 * T, G)
    _dual_equal(m, x, offs, ld, row_idx)


def test_dual_no_rows():
    m = require_gpu()
    x = np.zeros((0, 64), np.uint16)
    offs = np.zeros(4, np.int32)
    ld = oracle.mx_colwise_ld_min(0, 3)
    q, s, qT, sT = m.mx_quantize_dual(dev(np.zeros((1, 64), np.uint16))[:0], dev(offs), ld=ld)
    qo, so, qTo, sTo = oracle.mx_quantize_dual(x, offs, ld)
    assert q.numel() == 0 and s.numel() == 0
    assert np.array_equal(host(qT), qTo) and np.array_equal(host(sT), sTo)


def test_dual_full_size_sampled():
    """DeepSeek-V3-671B shard, gate+up X [65536, 7168]: the fused launch at full size, sampled rows
    (row-wise) and columns (column-wise) against the oracle."""
    m = require_gpu()
    lay = make_workload("dsv3_671b_shard", layers=["gate_up"]).layers[0]
    rng = np.random.default_rng(28)
    rows = np.concatenate([[0, lay.M - 1], rng.choice(lay.M, 300, replace=False)])
    cols = np.concatenate([[0, lay.K - 1], rng.choice(lay.K, 40, replace=False)])
    qro, sro = oracle.mx_quantize_rowwise(lay.x[rows])
    x = dev(lay.x)
    # the minimum row pitch and the recommended one the benchmark uses
    for ld in (oracle.mx_colwise_ld_min(lay.M, lay.G), m.mx_colwise_ld(lay.M, lay.G)):
        q, s, qT, sT = m.mx_quantize_dual(x, dev(lay.offs), ld=ld)
        assert np.array_equal(host(q[rows]), qro) and np.array_equal(host(s[rows]), sro)
        qo, so = oracle.mx_quantize_colwise(np.ascontiguousarray(lay.x[:, cols]), lay.offs, ld)
        assert np.array_equal(host(qT[cols]), qo) and np.array_equal(host(sT[cols]), so)
        del q, s, qT, sT


def test_blockwise_colwise_ragged_groups():
    """128-token column-wise blockwise copies (the blockwise wgrad operands): codes and fp32 scales
    bit-exact, ragged experts (empty, 1, 5, 130, 300 rows), extra tail columns, one group."""
    m = require_gpu()
    rng = np.random.default_rng(29)
    sizes = [0, 5, 130, 1, 300, 128, 0]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offs[-1])
    for C in (128, 384):
        x = random_bf16(rng, (M, C), outlier_frac=0.01, outlier_mult=1000.0)
        x[5:135, :128] = 0                      # an all-zero block: scale 1, zero codes
        for extra in (0, 128):
            ld = oracle.bw_colwise_ld_min(M, len(sizes)) + extra
            qT, sT = m.fp8bw_quantize_colwise_128(dev(x), dev(offs), ld=ld)
            qo, so = oracle.bw_quantize_colwise_128(x, offs, ld)
            assert np.array_equal(host(sT), so), f"scale mismatch at {np.argwhere(host(sT) != so)[:5]}"
            assert np.array_equal(host(qT), qo), f"code mismatch at {np.argwhere(host(qT) != qo)[:5]}"
    x = random_bf16(rng, (300, 256))
    ld1 = oracle.bw_colwise_ld_min(300, 1)           # 512: admissible for the oracle's offsets form too
    qT, sT = m.fp8bw_quantize_colwise_128(dev(x), None, ld=ld1)
    qo, so = oracle.bw_quantize_colwise_128(x, np.array([0, 300]), ld1)
    assert np.array_equal(host(qT), qo) and np.array_equal(host(sT), so)
