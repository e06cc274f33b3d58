"""GPU edge cases: the largest expert count the library accepts (1024, most of them empty, so wgrad runs
past the size-ordered scheduling of the first 256 experts), the opt-in offsets validator, and work issued
on a non-default stream."""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_expert_mx_amd as mm
from gpu_util import dev, host, random_bf16, require_gpu
from test_gpu_gemm import _rand_layer, run_layer

pytestmark = pytest.mark.gpu

G_MAX = 1024


def _sparse_sizes(rng, G, busy, hi):
    sizes = np.zeros(G, np.int64)
    idx = rng.choice(G - 1, busy, replace=False)
    sizes[idx] = rng.integers(1, hi, busy)
    sizes[G - 1] = 33                               # last expert non-empty: its tail ends the batch
    return sizes, np.sort(idx)


def test_max_expert_count_quantisers():
    m = require_gpu()
    rng = np.random.default_rng(50)
    sizes, _ = _sparse_sizes(rng, G_MAX, 60, 90)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offs[-1])
    x = random_bf16(rng, (M, 256))
    ld = oracle.mx_colwise_ld_min(M, G_MAX)
    q, s, qT, sT = m.mx_quantize_dual(dev(x), dev(offs), ld=ld)
    rq, rs, rqT, rsT = oracle.mx_quantize_dual(x, offs, ld)
    for got, ref, name in ((q, rq, "q"), (s, rs, "s"), (qT, rqT, "qT"), (sT, rsT, "sT")):
        assert np.array_equal(host(got), ref), name
    qT2, sT2 = m.mx_quantize_colwise(dev(x), dev(offs), ld=ld)
    assert np.array_equal(host(qT2), rqT) and np.array_equal(host(sT2), rsT)


@pytest.mark.parametrize("fast", [False, True])
def test_max_expert_count_gemms(fast):
    m = require_gpu()
    rng = np.random.default_rng(51)
    sizes, busy = _sparse_sizes(rng, G_MAX, 40, 70)
    L = _rand_layer(rng, sizes, 256, 256)
    rows = np.unique(rng.choice(L.M, 64, replace=False))
    # a few busy experts from the far end of the size order, the first, and empty ones
    empty = np.flatnonzero(sizes == 0)
    groups = np.unique(np.concatenate([busy[:3], busy[-3:], [G_MAX - 1], empty[:2], empty[-2:]]))
    run_layer(m, L, rows=rows, wgrad_groups=groups, fast=fast)


def test_max_expert_count_empty_experts_get_zero_gradient():
    m = require_gpu()
    rng = np.random.default_rng(52)
    sizes, _ = _sparse_sizes(rng, G_MAX, 20, 50)
    L = _rand_layer(rng, sizes, 128, 128)
    offs_d = dev(L.offs)
    ld = oracle.mx_colwise_ld_min(L.M, L.G)
    qdyT, sdyT = m.mx_quantize_colwise(dev(L.dy), offs_d, ld=ld)
    qxT, sxT = m.mx_quantize_colwise(dev(L.x), offs_d, ld=ld)
    dw = torch.full((L.G, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    m.mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs_d, L.M, dw=dw)
    h = host(dw)
    assert not np.isnan(h).any()
    assert not h[sizes == 0].any()


def test_offsets_validator():
    require_gpu()
    mm.mxmoe_check_offsets(dev(np.array([0, 3, 3, 10], np.int32)), 10)
    mm.mxmoe_check_offsets(dev(np.zeros(G_MAX + 1, np.int32)), 0)
    for bad in ([0, 5, 3, 10], [1, 3, 5, 10], [0, 3, 5, 9], [0, 3, 5, 11]):
        with pytest.raises(mm.MxMoeError):
            mm.mxmoe_check_offsets(dev(np.array(bad, np.int32)), 10)


def test_side_stream():
    """Quantisers and GEMMs issued on a non-default stream give the default-stream results."""
    m = require_gpu()
    rng = np.random.default_rng(53)
    offs = dev(np.array([0, 100, 100, 300], np.int32))
    x, w = dev(random_bf16(rng, (300, 256))), dev(random_bf16(rng, (3 * 256, 256), 0.05))
    qx, sx = m.mx_quantize_rowwise(x)
    qw, sw = m.mx_quantize_rowwise(w)
    qxT, sxT = m.mx_quantize_colwise(x, offs)
    y0 = m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs, 256)
    dw0 = m.mx_grouped_gemm_wgrad(qxT, sxT, qxT, sxT, offs, 300)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qx1, sx1 = m.mx_quantize_rowwise(x, stream=s)
        qxT1, sxT1 = m.mx_quantize_colwise(x, offs, stream=s)
        y1 = m.mx_grouped_gemm_fwd(qx1, sx1, qw, sw, offs, 256, stream=s)
        dw1 = m.mx_grouped_gemm_wgrad(qxT1, sxT1, qxT1, sxT1, offs, 300, stream=s)
    s.synchronize()
    assert torch.equal(qx1, qx) and torch.equal(sx1, sx)
    assert torch.equal(qxT1, qxT) and torch.equal(sxT1, sxT)
    assert torch.equal(y1, y0) and torch.equal(dw1, dw0)
