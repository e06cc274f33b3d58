"""Grouped GEMMs of a dropless MoE expert layer, in float64 (oracle).

iitak.ru, "NVIDIA sped up training of mixture-of-experts models on JAX
tenfold": every token is processed by its expert however uneven the load, and
the grouped GEMM runs all experts in one call, each on its real token count
(no padding to a capacity, no dropping).  opensourcebeat.com, "Enabling up to
41 % faster pre-training ...", section "Two-sided attack": MXFP8 is applied to
these grouped GEMMs.

Notation: G experts, int32 offsets offs[G+1] (offs[0] = 0, non-decreasing,
offs[G] = M), m_g = offs[g+1] - offs[g]; rows of X [M, K] and dY [M, N] are
sorted by expert; W is [G, N, K] (stored as [G*N, K]) and Y_g = X_g W_g^T.
DQ() is the exact value of a quantised operand.

* forward : Y[r, n]   = sum_k DQ(X)[r, k] DQ(W)[gN + n, k]            (r in group g)
* dgrad   : dX[r, k]  = sum_n DQ(dY)[r, n] DQ(W^c)[k, gN + n]         (W^c: W quantised
            column-wise, blocks along N)
* wgrad   : dW_g[n,k] = sum_{j < m_g} DQ(dY^c)[n, c_g + j] DQ(X^c)[k, c_g + j]
            (column-wise copies, group g starting at column c_g; dW_g = 0 for an
            empty group).  Blockwise: the same sum promoted per 128-token block,
            each block's partial multiplied by the dY row scale and the X row scale
            of that block.

Blockwise recipe (aifind.ru DeepSeek-V3 article, section "Low-precision
training: FP8 Framework"): the FP8 products over each 128-element slice of the
contraction are summed first and then promoted, i.e. multiplied by the
activation-tile scale and the weight-block scale and added to the running sum
(done exactly here, in float64).

Each group is a plain float64 matrix product of the dequantised operands
(np.matmul); every dequantised value and every product is exact in float64.
Row chunks keep host memory bounded.

Tolerance (not from the pages, which give none): |gpu - ref| <= 1e-5 *
sum_k |a_k b_k| per element, a and b the dequantised operands; for a bf16
output the GPU value may in addition be off by half a bf16 ulp of
(|ref| + that bound), since it is the bf16 rounding of an fp32 value.
"""
from __future__ import annotations

import numpy as np

from .blockwise import TILE, bw_group_columns
from .codecs import e4m3_decode
from .mx import BLOCK, mx_dequantize, mx_group_columns, mxfp4_dequantize

CHUNK = 4096
REL_TOL = 1e-5


def _rows_and_groups(offs, M, rows):
    offs = np.asarray(offs, dtype=np.int64)
    if offs[0] != 0 or offs[-1] != M or np.any(np.diff(offs) < 0):
        raise ValueError("bad offsets")
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    grp = np.searchsorted(offs, rows, side="right") - 1
    return rows, grp


def _grouped_rows(qa, sa, offs, rows, b_of_group, nout, deq_a):
    """out[i] = A[rows[i]] @ B_g^T for the group g of rows[i]; also sum |a b|."""
    rows, grp = _rows_and_groups(offs, qa.shape[0], rows)
    out = np.zeros((len(rows), nout))
    bound = np.zeros((len(rows), nout))
    for g in np.unique(grp):
        sel = np.flatnonzero(grp == g)
        B = b_of_group(int(g))                     # [nout, L] float64
        absB = np.abs(B)
        for c in range(0, len(sel), CHUNK):
            idx = sel[c:c + CHUNK]
            A = deq_a(rows[idx])                   # [n, L]
            out[idx] = A @ B.T
            bound[idx] = np.abs(A) @ absB.T
    return out, bound


def mx_gemm_fwd(qx, sx, qw, sw, offs, N, rows=None):
    """Forward grouped GEMM; returns (Y[rows], bound[rows]) in float64."""
    qx, sx, qw, sw = map(np.asarray, (qx, sx, qw, sw))
    return _grouped_rows(
        qx, sx, offs, rows,
        lambda g: mx_dequantize(qw[g * N:(g + 1) * N], sw[g * N:(g + 1) * N]),
        N, lambda r: mx_dequantize(qx[r], sx[r]))


def mx_gemm_dgrad(qdy, sdy, qwT, swT, offs, N, K, rows=None):
    """Data-gradient grouped GEMM; qwT/swT is W [G*N, K] quantised column-wise
    with uniform offsets g*N, i.e. [K, ldw] with group g at columns [gN, gN+N)."""
    qdy, sdy, qwT, swT = map(np.asarray, (qdy, sdy, qwT, swT))
    def b_of(g):
        c = g * N
        return mx_dequantize(qwT[:K, c:c + N], swT[:K, c // BLOCK:(c + N) // BLOCK])
    return _grouped_rows(qdy, sdy, offs, rows, b_of, K,
                         lambda r: mx_dequantize(qdy[r], sdy[r]))


def mx_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, N, K, groups=None, n_idx=None, k_idx=None):
    """Weight-gradient grouped GEMM over each group's own token columns.

    Returns (dW [len(groups), len(n_idx), len(k_idx)], bound) in float64.
    """
    qdyT, sdyT, qxT, sxT = map(np.asarray, (qdyT, sdyT, qxT, sxT))
    offs = np.asarray(offs, dtype=np.int64)
    G = len(offs) - 1
    groups = np.arange(G) if groups is None else np.asarray(groups)
    n_idx = np.arange(N) if n_idx is None else np.asarray(n_idx)
    k_idx = np.arange(K) if k_idx is None else np.asarray(k_idx)
    col0, nb = mx_group_columns(offs)
    out = np.zeros((len(groups), len(n_idx), len(k_idx)))
    bound = np.zeros_like(out)
    for i, g in enumerate(groups):
        m = int(offs[g + 1] - offs[g])
        if m == 0:
            continue
        c0 = int(col0[g])
        nblk = int(nb[g])
        sl = slice(c0 // BLOCK, c0 // BLOCK + nblk)
        A = mx_dequantize(qdyT[n_idx, c0:c0 + BLOCK * nblk], sdyT[n_idx, sl])[:, :m]
        B = mx_dequantize(qxT[k_idx, c0:c0 + BLOCK * nblk], sxT[k_idx, sl])[:, :m]
        out[i] = A @ B.T
        bound[i] = np.abs(A) @ np.abs(B).T
    return out, bound


# ---------------------------------------------------------------------------------- MXFP4 GEMMs
# The same three products over MXFP4 operands (E2M1 codes packed two per byte along the contraction
# axis, E8M0 per 32): packed column c covers elements 2c and 2c + 1.

def mxfp4_gemm_fwd(qx, sx, qw, sw, offs, N, rows=None):
    qx, sx, qw, sw = map(np.asarray, (qx, sx, qw, sw))
    return _grouped_rows(
        qx, sx, offs, rows,
        lambda g: mxfp4_dequantize(qw[g * N:(g + 1) * N], sw[g * N:(g + 1) * N]),
        N, lambda r: mxfp4_dequantize(qx[r], sx[r]))


def mxfp4_gemm_dgrad(qdy, sdy, qwT, swT, offs, N, K, rows=None):
    qdy, sdy, qwT, swT = map(np.asarray, (qdy, sdy, qwT, swT))
    def b_of(g):
        c = g * N
        return mxfp4_dequantize(qwT[:K, c // 2:(c + N) // 2], swT[:K, c // BLOCK:(c + N) // BLOCK])
    return _grouped_rows(qdy, sdy, offs, rows, b_of, K, lambda r: mxfp4_dequantize(qdy[r], sdy[r]))


def mxfp4_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, N, K, groups=None, n_idx=None, k_idx=None):
    qdyT, sdyT, qxT, sxT = map(np.asarray, (qdyT, sdyT, qxT, sxT))
    offs = np.asarray(offs, dtype=np.int64)
    G = len(offs) - 1
    groups = np.arange(G) if groups is None else np.asarray(groups)
    n_idx = np.arange(N) if n_idx is None else np.asarray(n_idx)
    k_idx = np.arange(K) if k_idx is None else np.asarray(k_idx)
    col0, nb = mx_group_columns(offs)
    out = np.zeros((len(groups), len(n_idx), len(k_idx)))
    bound = np.zeros_like(out)
    for i, g in enumerate(groups):
        m = int(offs[g + 1] - offs[g])
        if m == 0:
            continue
        c0, nblk = int(col0[g]), int(nb[g])
        sl = slice(c0 // BLOCK, c0 // BLOCK + nblk)
        bs = slice(c0 // 2, (c0 + BLOCK * nblk) // 2)
        A = mxfp4_dequantize(qdyT[n_idx, bs], sdyT[n_idx, sl])[:, :m]
        B = mxfp4_dequantize(qxT[k_idx, bs], sxT[k_idx, sl])[:, :m]
        out[i] = A @ B.T
        bound[i] = np.abs(A) @ np.abs(B).T
    return out, bound


def _bw_rows(qa, sa, offs, rows, b_of_group, nout):
    """Blockwise: promote each 128-slice partial sum with its two fp32 scales."""
    rows, grp = _rows_and_groups(offs, qa.shape[0], rows)
    L = qa.shape[1]
    out = np.zeros((len(rows), nout))
    bound = np.zeros((len(rows), nout))
    for g in np.unique(grp):
        sel = np.flatnonzero(grp == g)
        qb, sb = b_of_group(int(g))        # qb codes decoded [nout, L]; sb [nout, L/128]
        for c in range(0, len(sel), CHUNK):
            idx = sel[c:c + CHUNK]
            A = e4m3_decode(qa[rows[idx]])             # [n, L]
            As = np.asarray(sa[rows[idx]], dtype=np.float64)
            acc = np.zeros((len(idx), nout))
            bnd = np.zeros((len(idx), nout))
            for kb in range(L // TILE):
                ks = slice(kb * TILE, (kb + 1) * TILE)
                partial = A[:, ks] @ qb[:, ks].T          # unscaled 128-slice sum
                scale = As[:, kb:kb + 1] * sb[None, :, kb]
                acc += scale * partial
                bnd += np.abs(scale) * (np.abs(A[:, ks]) @ np.abs(qb[:, ks]).T)
            out[idx] = acc
            bound[idx] = bnd
    return out, bound


def bw_gemm_fwd(qx, sx, qw, sw, offs, N, rows=None):
    """Blockwise forward: qx [M,K] + sx f32 [M,K/128]; qw [G*N,K] + sw f32 [G*N/128, K/128]."""
    qx, sx, qw, sw = map(np.asarray, (qx, sx, qw, sw))
    def b_of(g):
        qb = e4m3_decode(qw[g * N:(g + 1) * N])
        sb = np.repeat(np.asarray(sw, dtype=np.float64)[g * N // TILE:(g + 1) * N // TILE], TILE, axis=0)
        return qb, sb
    return _bw_rows(qx, sx, offs, rows, b_of, N)


def bw_gemm_dgrad(qdy, sdy, qw, sw, offs, N, K, rows=None):
    """Blockwise dgrad: dX[r,k] = sum_nb sdy[r,nb] sw[gN/128+nb, k/128] sum_{n in nb} qdy[r,n] qw[gN+n,k].

    dY is quantised 1x128 along N (sdy [M, N/128]); the 128x128 weight blocks of
    the forward pass are reused, read transposed.
    """
    qdy, sdy, qw, sw = map(np.asarray, (qdy, sdy, qw, sw))
    sw64 = np.asarray(sw, dtype=np.float64)
    def b_of(g):
        qb = e4m3_decode(qw[g * N:(g + 1) * N]).T                       # [K, N]
        sb = np.repeat(sw64[g * N // TILE:(g + 1) * N // TILE].T, TILE, axis=0)   # [K, N/128]
        return qb, sb
    return _bw_rows(qdy, sdy, offs, rows, b_of, K)


def bw_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, N, K, groups=None, n_idx=None, k_idx=None):
    """Blockwise weight gradient: dW_g[n,k] = sum_b sdyT[n, b] sxT[k, b] sum_{j in block b} qdyT[n, j] qxT[k, j]
    over group g's 128-token blocks b (columns from bw_group_columns; pads hold zero codes).

    Returns (dW [len(groups), len(n_idx), len(k_idx)], bound) in float64.
    """
    qdyT, qxT = np.asarray(qdyT), np.asarray(qxT)
    sdyT, sxT = np.asarray(sdyT, dtype=np.float64), np.asarray(sxT, dtype=np.float64)
    offs = np.asarray(offs, dtype=np.int64)
    G = len(offs) - 1
    groups = np.arange(G) if groups is None else np.asarray(groups)
    n_idx = np.arange(N) if n_idx is None else np.asarray(n_idx)
    k_idx = np.arange(K) if k_idx is None else np.asarray(k_idx)
    col0, nb = bw_group_columns(offs)
    out = np.zeros((len(groups), len(n_idx), len(k_idx)))
    bound = np.zeros_like(out)
    for i, g in enumerate(groups):
        c0 = int(col0[g])
        for b in range(int(nb[g])):
            cs = slice(c0 + TILE * b, c0 + TILE * (b + 1))
            A = e4m3_decode(qdyT[n_idx, cs])
            B = e4m3_decode(qxT[k_idx, cs])
            scale = sdyT[n_idx, c0 // TILE + b][:, None] * sxT[k_idx, c0 // TILE + b][None, :]
            out[i] += scale * (A @ B.T)
            bound[i] += np.abs(scale) * (np.abs(A) @ np.abs(B).T)
    return out, bound


def _ulp_bf16(x):
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(np.where(x > 0, x, 1.0))
    return np.where(x > 0, np.ldexp(1.0, ex - 1 - 7), 0.0)


def gemm_tolerance(ref, bound, out_dtype: str = "f32", rel: float = REL_TOL):
    """Per-element admissible |gpu - ref|."""
    tol = rel * np.asarray(bound, dtype=np.float64)
    if out_dtype == "bf16":
        tol = tol + 0.5 * _ulp_bf16(np.abs(ref) + tol)
    elif out_dtype != "f32":
        raise ValueError(out_dtype)
    return tol


def check_gemm(got, ref, bound, out_dtype: str = "f32", rel: float = REL_TOL):
    """Returns (all_ok, worst |err|/tol, index of the worst element)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = gemm_tolerance(ref, bound, out_dtype, rel)
    err = np.abs(got - ref)
    if not np.all(np.isfinite(got)):
        return False, np.inf, int(np.flatnonzero(~np.isfinite(got).reshape(-1))[0])
    ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = int(np.argmax(ratio)) if ratio.size else 0
    r = float(ratio.reshape(-1)[worst]) if ratio.size else 0.0
    return bool(r <= 1.0), r, worst

