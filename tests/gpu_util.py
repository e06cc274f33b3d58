"""Helpers shared by the GPU parity tests (host <-> device copies, seeded inputs)."""
import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_moe_expert_mx_amd as m
    m.lib()          # raises if the library is not built: GPU tests never fall back
    return m


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor with the same bytes (uint16 bf16 patterns go to int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def random_bf16(rng, shape, std=1.0, outlier_frac=0.0, outlier_mult=100.0):
    from workloads import f32_to_bf16_bits
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outlier_frac:
        idx = rng.choice(x.size, int(outlier_frac * x.size) or 1, replace=False)
        x.reshape(-1)[idx] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def same_bytes(got, ref, what):
    """Quantiser outputs of the GPU (codes, scales, ...) equal the oracle's, element by element."""
    for i, (g, r) in enumerate(zip(got, ref)):
        g, r = np.asarray(g), np.asarray(r)
        assert g.shape == r.shape and np.array_equal(g, r), f"{what}: output {i} differs from the oracle's quantisation"


def check_rows(n, idx=None, seed=0, cap=256):
    """Operand rows whose bytes are compared with the oracle's quantisation before they feed an oracle
    GEMM: the given ones, else all up to `cap`, else `cap` seeded ones including the first and last."""
    if idx is not None:
        return np.asarray(idx, np.int64)
    if n <= cap:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, cap - 2, replace=False)]))
