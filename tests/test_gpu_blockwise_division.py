"""GPU parity of the blockwise quantisers' element division with fp32 scales s = fl32(amax / 448): the
kernels form fl32(v / s) from one reciprocal per tile and two FMAs (falling back to a division per
element for tiles with amax below 2^-59), and the codes must equal the oracle's, which divides in
IEEE fp32 (aifind.ru DeepSeek-V3 article, section "Low-precision training: FP8 Framework", figure
caption (a): 1x128 activation tiles, 128x128 weight blocks).  Every finite bf16 magnitude is a 1x128
tile's amax; its other elements are drawn uniformly over the bit patterns below it, so every binade
down to the subnormals (quotients that underflow) is hit, with -0 and the largest non-maximal value."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, require_gpu
from workloads import f32_to_bf16_bits, routing_offsets

pytestmark = pytest.mark.gpu


def _equal(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what} mismatch at {bad[:5]}: gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]}"


def _tiles_below(rng, amax_bits, n):
    """[len(amax_bits), n] bf16 patterns: element 0 is the tile's amax (negative in odd tiles), element 1
    is -0, element 2 the next magnitude down, the rest uniform over the magnitudes below amax with random
    signs."""
    a = amax_bits.astype(np.uint32)[:, None]
    t = (rng.integers(0, 1 << 32, (len(amax_bits), n), dtype=np.uint64) % (a + 1)).astype(np.uint32)
    t |= (rng.integers(0, 2, t.shape, dtype=np.uint32) << 15)
    t[:, 0] = amax_bits
    t[1::2, 0] |= 0x8000
    t[:, 1] = 0x8000
    t[:, 2] = np.maximum(amax_bits.astype(np.int64) - 1, 0).astype(np.uint32)
    return t.astype(np.uint16)


def test_act_every_bf16_magnitude_as_tile_amax():
    m = require_gpu()
    rng = np.random.default_rng(70)
    mags = np.arange(1, 0x7F80, dtype=np.uint32)
    x = _tiles_below(rng, mags, 128)
    q, s = m.fp8bw_quantize_act_1x128(dev(x))
    qo, so = oracle.bw_quantize_act_1x128(x)
    _equal(host(s), so, "scale")
    _equal(host(q), qo, "code")


def test_weight_blocks_from_tiny_to_huge_amax():
    m = require_gpu()
    rng = np.random.default_rng(71)
    nb_r, nb_c = 12, 16                                           # 192 blocks of 128 x 128
    amax_bits = np.linspace(1, 0x7F7F, nb_r * nb_c).astype(np.uint32)
    amax_bits[:8] = [1, 0x0080, 0x1000, 0x2180, 0x21FF, 0x2200, 0x2201, 0x3F80]   # around 2^-59 = 0x2200
    w = np.empty((128 * nb_r, 128 * nb_c), np.uint16)
    for b, a in enumerate(amax_bits):
        i, j = divmod(b, nb_c)
        blk = _tiles_below(rng, np.full(128, a, np.uint32), 128)
        w[128 * i:128 * i + 128, 128 * j:128 * j + 128] = rng.permutation(blk.reshape(-1)).reshape(128, 128)
    q, s, qT = m.fp8bw_quantize_weight_128x128(dev(w), transposed=True)
    qo, so = oracle.bw_quantize_weight_128x128(w)
    _equal(host(s), so, "weight scale")
    _equal(host(q), qo, "weight code")
    _equal(host(qT), qo.T, "transposed weight code")


def test_colwise_blocks_from_tiny_to_huge_amax():
    m = require_gpu()
    rng = np.random.default_rng(72)
    sizes = [130, 0, 7, 256, 45]
    offs = routing_offsets(sizes)
    M, C = int(offs[-1]), 512
    # column j spans a 2^+-4 range around 2^e_j, e_j from -132 to 120: column blocks with a tiny
    # (per-element division) and a normal (FMA) amax side by side
    e = np.linspace(-132, 120, C).round().astype(np.int32)
    u = rng.uniform(-16.0, 16.0, (M, C)).astype(np.float64) * np.exp2(e.astype(np.float64))[None, :]
    x = f32_to_bf16_bits(u.astype(np.float32))
    x[0, :] = 0x8000                                             # -0 in every column
    ld = oracle.bw_colwise_ld_min(M, len(sizes))
    qT, sT = m.fp8bw_quantize_colwise_128(dev(x), dev(offs), ld=ld)
    qo, so = oracle.bw_quantize_colwise_128(x, offs, ld)
    _equal(host(sT), so, "colwise scale")
    _equal(host(qT), qo, "colwise code")
