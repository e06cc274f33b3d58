"""Seeded synthetic routed-token workloads for the MXFP8 expert-GEMM path.

This module only draws inputs: group sizes (the per-expert token counts of a
dropless MoE layer) and bf16 tensors.  It contains none of the method's
arithmetic (no quantisation, no GEMM) and is shared by the CPU oracle side
(tests, bench baseline) and the GPU side (tests, bench, smoke) so that both
see the same bytes.

Shapes and distributions stand in for the workloads the pages describe
(DeepSeek-V3 and Llama-4-Scout expert layers; the pages publish no data set):

* tiny     -- 4 experts, K=256, N=512, 1024 routed rows, one empty expert,
              N(0,1) values with 0.1 % of entries multiplied by 100.
* dsv3_16b -- 64 experts, 8192 tokens x top-6 = 49152 rows, group sizes from
              the top-6 of a softmax over N(0,1) router logits; gate+up
              (N=2816, K=2048) and down (N=2048, K=1408) layers;
              activations N(0,1), weights N(0, 0.02^2).
* dsv3_671b_shard -- 8 local experts of a 256-expert layer, 65536 rows, one
              expert with 17 rows and the rest Zipf(s=1.2)-skewed; gate+up
              (N=4096, K=7168) and down (N=7168, K=2048); 0.1 % of entries
              multiplied by 10^u, u ~ U(1, 3).
* llama4_scout -- 16 experts, top-1, 32768 rows, Dirichlet(5) fractions;
              gate+up (N=16384, K=5120) and down (N=5120, K=8192); N(0,1).

Floats are drawn as float32 and rounded to bfloat16 with round-to-nearest-even
on the bit pattern; tensors are returned as uint16 bit arrays.  Large tensors
are drawn in fixed chunks of 2^22 elements, each from its own child of the
workload's SeedSequence, and filled by a thread pool: the bytes depend only on
the seed, never on the number of threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["Layer", "Workload", "f32_to_bf16_bits", "make_workload", "WORKLOADS",
           "routing_offsets", "make_layer", "random_offsets"]


CHUNK = 1 << 22          # elements per independently seeded chunk


def _threads() -> int:
    # the host share of one GPU is at most 16 cores
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _parallel(fn, n: int) -> None:
    if n <= 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(max_workers=min(_threads(), n)) as ex:
        list(ex.map(fn, range(n)))


def _round_chunk(src: np.ndarray, dst: np.ndarray) -> None:
    if not np.all(np.isfinite(src)):
        raise ValueError("non-finite input")
    u = src.view(np.uint32)
    r = u >> 16
    r &= 1
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    dst[...] = r


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf, of = x.reshape(-1), out.reshape(-1)
    n = xf.size
    _parallel(lambda i: _round_chunk(xf[i * CHUNK:(i + 1) * CHUNK], of[i * CHUNK:(i + 1) * CHUNK]),
              -(-n // CHUNK))
    return out


@dataclass
class Layer:
    """One expert linear layer: Y_g = X_g W_g^T for every expert g.

    x  : uint16 [M, K] bf16 bits, rows sorted by expert
    w  : uint16 [G, N, K] bf16 bits
    dy : uint16 [M, N] bf16 bits (the upstream gradient)
    offs : int32 [G+1], offs[0] = 0, non-decreasing, offs[G] = M
    """
    name: str
    G: int
    M: int
    N: int
    K: int
    offs: np.ndarray
    x: np.ndarray
    w: np.ndarray
    dy: np.ndarray

    @property
    def sizes(self) -> np.ndarray:
        return np.diff(self.offs)


@dataclass
class Workload:
    name: str
    seed: int
    layers: List[Layer] = field(default_factory=list)
    description: str = ""


def _normal(seq: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) of the given shape, chunk i drawn from child i of `seq`."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n = flat.size
    nchunks = -(-n // CHUNK)
    kids = seq.spawn(nchunks)

    def fill(i):
        part = flat[i * CHUNK:(i + 1) * CHUNK]
        np.random.Generator(np.random.PCG64(kids[i])).standard_normal(out=part, dtype=np.float32)
        if std != 1.0:
            part *= np.float32(std)

    _parallel(fill, nchunks)
    return out


def _outliers(rng: np.random.Generator, a: np.ndarray, frac: float, mode: str) -> None:
    """Multiply a uniformly chosen fraction of entries (without replacement) in place."""
    n = a.size
    k = int(round(frac * n))
    if k == 0:
        return
    idx = rng.choice(n, size=k, replace=False)
    flat = a.reshape(-1)
    if mode == "x100":
        flat[idx] *= np.float32(100.0)
    elif mode == "pow10":
        u = rng.uniform(1.0, 3.0, size=k).astype(np.float32)
        flat[idx] *= np.power(np.float32(10.0), u).astype(np.float32)
    else:
        raise ValueError(mode)


def routing_offsets(sizes) -> np.ndarray:
    sizes = np.asarray(sizes, dtype=np.int64)
    offs = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=offs[1:])
    return offs.astype(np.int32)


def _sizes_tiny(rng):
    s = rng.multinomial(1024, [1 / 3, 1 / 3, 1 / 3, 0.0])
    s[3] = 0
    return s


def _sizes_top6(rng, tokens=8192, experts=64, topk=6):
    logits = rng.standard_normal(size=(tokens, experts), dtype=np.float32)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    # top-k with ties broken toward the lower expert index (stable sort on -p)
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    return np.bincount(order.reshape(-1), minlength=experts)


def _sizes_zipf_shard(rng, rows=65536, experts=8, tiny=17, s=1.2):
    tiny_idx = int(rng.integers(0, experts))
    ranks = np.arange(1, experts, dtype=np.float64)
    w = ranks ** (-s)
    w /= w.sum()
    counts = rng.multinomial(rows - tiny, w)
    perm = rng.permutation(experts - 1)
    others = [e for e in range(experts) if e != tiny_idx]
    sizes = np.zeros(experts, dtype=np.int64)
    sizes[tiny_idx] = tiny
    for rank_pos, e in zip(perm, others):
        sizes[e] = counts[rank_pos]
    return sizes


def _sizes_dirichlet(rng, rows=32768, experts=16, alpha=5.0):
    frac = rng.dirichlet(np.full(experts, alpha))
    return rng.multinomial(rows, frac)


def make_layer(rng, name, sizes, N, K, x_std=1.0, w_std=1.0, dy_std=1.0,
               outliers: Optional[str] = None, outlier_frac=1e-3) -> Layer:
    """One layer's tensors; `rng` supplies the layer's seed and the outlier positions."""
    offs = routing_offsets(sizes)
    G = len(sizes)
    M = int(offs[-1])
    seq = np.random.SeedSequence(int(rng.integers(0, 2 ** 63)))
    sx, sw, sdy = seq.spawn(3)
    x = _normal(sx, (M, K), x_std)
    w = _normal(sw, (G, N, K), w_std)
    dy = _normal(sdy, (M, N), dy_std)
    if outliers is not None:
        for a in (x, w, dy):
            _outliers(rng, a, outlier_frac, outliers)
    xb = f32_to_bf16_bits(x)
    del x
    wb = f32_to_bf16_bits(w)
    del w
    return Layer(name, G, M, N, K, offs, xb, wb, f32_to_bf16_bits(dy))


def random_offsets(rng, M: int, G: int, empty_frac: float = 0.25) -> np.ndarray:
    """Ragged group sizes summing to M with some empty groups (for edge-case tests)."""
    w = rng.random(G)
    w[rng.random(G) < empty_frac] = 0.0
    if w.sum() == 0:
        w[0] = 1.0
    sizes = rng.multinomial(M, w / w.sum())
    return routing_offsets(sizes)


# (layer, routed rows M, N, K) of each workload, as make_workload builds them (no data generated)
_SHAPES: Dict[str, List[Tuple[str, int, int, int]]] = {
    "tiny": [("single", 1024, 512, 256)],
    "dsv3_16b": [("gate_up", 49152, 2816, 2048), ("down", 49152, 2048, 1408)],
    "dsv3_671b_shard": [("gate_up", 65536, 4096, 7168), ("down", 65536, 7168, 2048)],
    "llama4_scout": [("gate_up", 32768, 16384, 5120), ("down", 32768, 5120, 8192)],
}
_SHAPES["dsv3_16b_blockwise"] = _SHAPES["dsv3_16b"]


def layer_shapes(name: str) -> List[Tuple[str, int, int, int]]:
    """(layer, M, N, K) of a named workload's layers without generating its tensors."""
    return list(_SHAPES[name])


def make_workload(name: str, layers: Optional[List[str]] = None) -> Workload:
    """Build a named workload.  `layers` selects a subset ("gate_up", "down")."""
    if name == "tiny":
        rng = np.random.default_rng(101)
        sizes = _sizes_tiny(rng)
        wl = Workload(name, 101, description="4 experts, K=256, N=512, 1024 rows (512 tokens top-2), expert 3 empty")
        wl.layers.append(make_layer(rng, "single", sizes, 512, 256, outliers="x100"))
        return wl
    if name in ("dsv3_16b", "dsv3_16b_blockwise"):
        rng = np.random.default_rng(102)
        sizes = _sizes_top6(rng)
        wl = Workload(name, 102, description="64 experts, 8192 tokens top-6 = 49152 rows")
        want = layers or ["gate_up", "down"]
        lay = make_layer(rng, "gate_up", sizes, 2816, 2048, w_std=0.02)
        if "gate_up" in want:
            wl.layers.append(lay)
        del lay
        lay = make_layer(rng, "down", sizes, 2048, 1408, w_std=0.02)
        if "down" in want:
            wl.layers.append(lay)
        return wl
    if name == "dsv3_671b_shard":
        rng = np.random.default_rng(103)
        sizes = _sizes_zipf_shard(rng)
        wl = Workload(name, 103, description="8 local experts, 65536 rows, Zipf(1.2) sizes with one 17-row expert")
        want = layers or ["gate_up", "down"]
        lay = make_layer(rng, "gate_up", sizes, 4096, 7168, w_std=0.02, outliers="pow10")
        if "gate_up" in want:
            wl.layers.append(lay)
        del lay
        if "down" in want:
            wl.layers.append(make_layer(rng, "down", sizes, 7168, 2048, w_std=0.02, outliers="pow10"))
        return wl
    if name == "llama4_scout":
        rng = np.random.default_rng(104)
        sizes = _sizes_dirichlet(rng)
        wl = Workload(name, 104, description="16 experts, top-1, 32768 rows, Dirichlet(5) fractions")
        want = layers or ["gate_up", "down"]
        lay = make_layer(rng, "gate_up", sizes, 16384, 5120)
        if "gate_up" in want:
            wl.layers.append(lay)
        del lay
        if "down" in want:
            wl.layers.append(make_layer(rng, "down", sizes, 5120, 8192))
        return wl
    raise KeyError(name)


WORKLOADS: Dict[str, str] = {
    "tiny": "4 experts, hidden 256, expert N 512, 1024 routed rows",
    "dsv3_16b": "DeepSeek-V3-16B-shaped expert layers, 64 experts, 49152 rows",
    "dsv3_671b_shard": "DeepSeek-V3-671B one-GPU expert shard, 8 experts, 65536 rows",
    "llama4_scout": "Llama-4-Scout-shaped expert layers, 16 experts, 32768 rows",
    "dsv3_16b_blockwise": "the dsv3_16b tensors, for the blockwise-FP8 recipe",
}
