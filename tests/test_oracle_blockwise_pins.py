"""Discriminating pins of the blockwise (1x128 / 128x128) oracle, DeepSeek-V3 recipe (aifind.ru,
"DeepSeek-V3: a revolutionary high-performance language model with low training cost", section
"Low-precision training: FP8 Framework", captions (a) and (b)).

* The element step q = E4M3(fl32(v / s)) takes the float32 quotient, not the exact one.  Elements are
  searched on the host for which the two round to different E4M3 codes; the oracle's codes must equal
  torch's CPU float32 division followed by its float8_e4m3fn cast (library routines, independent of
  the oracle), and must differ from the codes of the exact quotient.
* The blockwise dgrad against the dense product of the dequantised operands, with every 1x128 dY scale
  and every 128x128 weight scale distinct, so that a misindexed or transposed scale grid fails.
"""
import numpy as np
import torch

from oracle import (bw_colwise_ld_min, bw_dequantize_act, bw_dequantize_weight, bw_gemm_dgrad,
                    bw_gemm_fwd, bw_quantize_act_1x128, bw_quantize_colwise_128, bw_quantize_weight_128x128,
                    e4m3_decode, e4m3_encode)
from workloads import routing_offsets


def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def _quotient_cases(n_amax=40):
    """(amax, v) float32 pairs (both bf16 values, 0 < v <= amax) whose float32 quotient v / s, with
    s = fl32(amax / 448), rounds to another E4M3 code than the exact quotient does."""
    pos = _bf16_value(np.arange(1, 0x7F80))
    cases = []
    for ab in np.arange(0x3E00, 0x4100, 5, dtype=np.uint32):        # amax from 0.125 to 8
        amax = _bf16_value(ab)
        s = np.float32(amax / np.float32(448.0))
        v = pos[pos <= amax]
        c32 = e4m3_encode((v / s).astype(np.float32).astype(np.float64))
        c64 = e4m3_encode(v.astype(np.float64) / np.float64(s))
        for i in np.flatnonzero(c32 != c64)[:2]:
            cases.append((np.float32(amax), np.float32(v[i])))
        if len(cases) >= n_amax:
            break
    return cases


def _torch_codes(v, s):
    """E4M3 codes of fl32(v / s) by torch: IEEE float32 division, then the float8_e4m3fn cast
    (round to nearest even; the quotients here stay below 464, where that cast is finite)."""
    q = torch.from_numpy(np.asarray(v, np.float32)) / torch.from_numpy(np.asarray(s, np.float32))
    assert float(q.abs().max()) < 464.0
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quotient_cases_exist_in_both_code_ranges():
    cases = _quotient_cases()
    assert len(cases) >= 20
    codes = [int(_torch_codes([v], [np.float32(a / np.float32(448))])[0]) for a, v in cases]
    assert min(codes) < 8 and max(codes) >= 8, codes       # subnormal and normal E4M3 codes


def test_act_1x128_codes_follow_the_fp32_quotient():
    cases = _quotient_cases()
    x = np.zeros((len(cases), 256), np.float32)
    for r, (amax, v) in enumerate(cases):
        x[r, 0] = amax                                   # tile 0: amax, +v, -v
        x[r, 5], x[r, 77] = v, -v
        x[r, 128 + 3] = -amax                            # tile 1: amax as a negative value, then v
        x[r, 128 + 100] = v
    q, s = bw_quantize_act_1x128(_bits(x))
    amax = np.array([a for a, _ in cases], np.float32)
    s_ref = (torch.from_numpy(amax) / torch.tensor(448.0, dtype=torch.float32)).numpy()
    assert np.array_equal(s[:, 0], s_ref) and np.array_equal(s[:, 1], s_ref)
    for r in range(len(cases)):
        for c in (0, 5, 77, 128 + 3, 128 + 100):
            want = _torch_codes([x[r, c]], [s_ref[r]])[0]
            assert q[r, c] == want, (r, c, q[r, c], want)
    # the exact quotient would give other codes for the searched elements
    v = np.array([v for _, v in cases], np.float64)
    exact = e4m3_encode(v / s_ref.astype(np.float64))
    assert np.all(exact != q[:, 5])


def test_weight_and_colwise_codes_follow_the_fp32_quotient():
    cases = _quotient_cases(8)
    # 128x128 weight blocks: block (i, j) holds case 2i + j's amax and v
    w = np.zeros((256, 256), np.float32)
    for idx, (amax, v) in enumerate(cases[:4]):
        i, j = divmod(idx, 2)
        w[128 * i + 7, 128 * j + 9] = amax
        w[128 * i + 100, 128 * j + 3] = v
        w[128 * i + 3, 128 * j + 120] = -v
    qw, sw = bw_quantize_weight_128x128(_bits(w))
    for idx, (amax, v) in enumerate(cases[:4]):
        i, j = divmod(idx, 2)
        s_ref = (torch.tensor(amax, dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32)).item()
        assert sw[i, j] == np.float32(s_ref)
        assert qw[128 * i + 100, 128 * j + 3] == _torch_codes([v], [s_ref])[0]
        assert qw[128 * i + 3, 128 * j + 120] == _torch_codes([-v], [s_ref])[0]
    # 128-token column-wise blocks: two experts, a short one (blocks restart at its first row)
    offs = routing_offsets([130, 40])
    M = int(offs[-1])
    x = np.zeros((M, 128), np.float32)
    for c, (amax, v) in enumerate(cases[:4]):
        r0 = 0 if c < 2 else 130                          # expert 0's first block, expert 1's only block
        x[r0 + 2, c], x[r0 + 30, c] = amax, v
    ld = bw_colwise_ld_min(M, 2)
    qT, sT = bw_quantize_colwise_128(_bits(x), offs, ld)
    for c, (amax, v) in enumerate(cases[:4]):
        col = 0 if c < 2 else 256                         # expert 1 starts at column 128 * ceil(130/128)
        s_ref = (torch.tensor(amax, dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32)).item()
        assert sT[c, col // 128] == np.float32(s_ref)
        assert qT[c, col + 30] == _torch_codes([v], [s_ref])[0]


def _distinct_scale_operands(rng, M, G, N, K):
    """Random E4M3 codes with every 1x128 dY scale and every 128x128 weight scale a distinct power of
    two (exact products), and no code NaN."""
    qdy = rng.integers(0, 0x7F, size=(M, N)).astype(np.uint8) | (rng.integers(0, 2, (M, N)) << 7).astype(np.uint8)
    qw = rng.integers(0, 0x7F, size=(G * N, K)).astype(np.uint8) | (rng.integers(0, 2, (G * N, K)) << 7).astype(np.uint8)
    n_sdy, n_sw = M * (N // 128), (G * N // 128) * (K // 128)
    e = rng.permutation(np.arange(-60, -60 + n_sdy + n_sw))
    sdy = np.ldexp(1.0, e[:n_sdy]).astype(np.float32).reshape(M, N // 128)
    sw = np.ldexp(1.0, e[n_sdy:]).astype(np.float32).reshape(G * N // 128, K // 128)
    return qdy, sdy, qw, sw


def test_bw_dgrad_equals_dense_product_with_distinct_scales():
    """dX_g = DQ(dY_g) DQ(W_g): the dense float64 product of the dequantised operands (dY scaled per
    1x128 tile along N, W per 128x128 block), with every scale distinct.  A per-expert W of 256 x 256
    has a 2 x 2 scale grid whose transpose has the same shape: the transposed reading must fail."""
    rng = np.random.default_rng(60)
    sizes, N, K = [3, 0, 5, 2], 256, 256
    offs = routing_offsets(sizes)
    M, G = int(offs[-1]), len(sizes)
    qdy, sdy, qw, sw = _distinct_scale_operands(rng, M, G, N, K)
    dx, bound = bw_gemm_dgrad(qdy, sdy, qw, sw, offs, N, K)
    D = bw_dequantize_act(qdy, sdy)                          # [M, N]
    Wd = bw_dequantize_weight(qw, sw)                        # [G*N, K]
    grp = np.repeat(np.arange(G), sizes)
    dense = np.stack([D[r] @ Wd[g * N:(g + 1) * N] for r, g in enumerate(grp)])
    assert np.all(np.abs(dx - dense) <= 1e-12 * bound)
    # the same dense product with each expert's weight-scale grid transposed (a plausible misreading
    # of the transposed weight blocks) is far outside that bound
    swt = sw.astype(np.float64).copy()
    nb = N // 128
    for g in range(G):
        swt[g * nb:(g + 1) * nb] = sw[g * nb:(g + 1) * nb].T
    Wt = e4m3_decode(qw) * np.repeat(np.repeat(swt, 128, 0), 128, 1)
    wrong = np.stack([D[r] @ Wt[g * N:(g + 1) * N] for r, g in enumerate(grp)])
    assert np.any(np.abs(wrong - dense) > 1e-3 * bound)
    # the forward pass with the same weights (X scales distinct too) against its dense product
    qx, sx, _, _ = _distinct_scale_operands(rng, M, G, K, N)
    y, ybound = bw_gemm_fwd(qx, sx, qw, sw, offs, N)
    X = bw_dequantize_act(qx, sx)
    dense_y = np.stack([X[r] @ Wd[g * N:(g + 1) * N].T for r, g in enumerate(grp)])
    assert np.all(np.abs(y - dense_y) <= 1e-12 * ybound)
