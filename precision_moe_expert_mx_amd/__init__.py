"""Python binding of libmxmoe (MXFP8 quantisers and dropless grouped GEMMs for MI355X / gfx950).

Argument marshalling only: every step runs in the HIP library.  Tensors are torch tensors on the
current HIP device (bf16 inputs may be given as torch.bfloat16 or as uint16/int16 bit patterns);
outputs are allocated with torch when not passed in.  Calls are asynchronous on torch's current
stream unless `stream` (a torch.cuda.Stream or a raw hipStream_t integer) is given.

The library must be built (``python -m precision_moe_expert_mx_amd.build``); importing this package
without it raises, and there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "LIB_PATH", "MxMoeError", "lib", "abi_version",
    "mx_colwise_ld_min", "mxmoe_pitch", "mx_colwise_ld", "mxfp4_colwise_ld",
    "mx_quantize_rowwise", "mx_quantize_colwise", "mx_quantize_dual",
    "mx_grouped_gemm_fwd", "mx_grouped_gemm_dgrad", "mx_grouped_gemm_wgrad", "mx_grouped_gemm_fwd_swiglu",
    "mx_quantize_rowwise_tiled", "mx_quantize_colwise_tiled", "mx_quantize_dual_tiled", "mx_grouped_gemm_fwd_tiled",
    "mx_grouped_gemm_fwd_swiglu_tiled", "mx_grouped_gemm_dgrad_tiled", "mx_grouped_gemm_wgrad_tiled",
    "fp8bw_quantize_act_1x128", "fp8bw_quantize_weight_128x128",
    "fp8bw_grouped_gemm_fwd", "fp8bw_grouped_gemm_dgrad", "mxmoe_check_offsets",
    "fp8bw_grouped_gemm_fwd_pow2", "fp8bw_grouped_gemm_dgrad_pow2", "fp8bw_grouped_gemm_wgrad_pow2",
    "fp8bw_colwise_ld_min", "fp8bw_quantize_colwise_128", "fp8bw_grouped_gemm_wgrad",
    "mxfp4_quantize_rowwise", "mxfp4_quantize_colwise", "mxfp4_grouped_gemm_fwd", "mxfp4_grouped_gemm_dgrad",
    "mxfp4_grouped_gemm_wgrad",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxmoe.so")

MXMOE_F32, MXMOE_BF16 = 0, 1
_STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_ALIGN", 4: "ERR_DTYPE", 5: "ERR_OFFSETS",
           6: "ERR_HIP", 7: "ERR_UNSUPPORTED"}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

# name -> (restype, argtypes); mirrors include/mxmoe.h
_SIGS = {
    "mxmoe_abi_version": (ctypes.c_int, []),
    "mxmoe_last_error": (ctypes.c_char_p, []),
    "mx_colwise_ld_min": (_i64, [_i64, _i32]),
    "mxmoe_pitch": (_i64, [_i64]),
    "mx_quantize_rowwise": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "mx_quantize_colwise": (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _i64, _p]),
    "mx_quantize_dual": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _p, _i32, _p, _p, _p, _p, _i64, _p]),
    "mx_grouped_gemm_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int, _p]),
    "mx_grouped_gemm_fwd_swiglu": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p,
                                                  _i64, _p]),
    "mx_grouped_gemm_dgrad": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int, _p]),
    "mx_grouped_gemm_wgrad": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int, _p]),
    "fp8bw_quantize_act_1x128": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "fp8bw_quantize_weight_128x128": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _p]),
    "fp8bw_grouped_gemm_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int, _p]),
    "fp8bw_grouped_gemm_dgrad": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int, _p]),
    "fp8bw_colwise_ld_min": (_i64, [_i64, _i32]),
    "mxfp4_quantize_rowwise": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "mxfp4_quantize_colwise": (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _i64, _p]),
    "mxfp4_grouped_gemm_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int, _p]),
    "mxfp4_grouped_gemm_dgrad": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int,
                                                _p]),
    "mxfp4_grouped_gemm_wgrad": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int,
                                                _p]),
    "fp8bw_quantize_colwise_128": (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _i64, _p]),
    "fp8bw_quantize_act_1x128_pow2": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "fp8bw_quantize_weight_128x128_pow2": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _p]),
    "fp8bw_quantize_colwise_128_pow2": (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _i64, _p]),
    "fp8bw_grouped_gemm_wgrad": (ctypes.c_int, [_p, _p, _p, _p, _i64, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_int,
                                                _p]),
    "mxmoe_check_offsets": (ctypes.c_int, [_p, _i32, _i64, _p]),
}
# the 128-byte tiled layouts: the same arguments as the row-major entry points
for _n in ("mx_quantize_rowwise", "mx_quantize_colwise", "mx_quantize_dual", "mx_grouped_gemm_fwd",
           "mx_grouped_gemm_fwd_swiglu", "mx_grouped_gemm_dgrad", "mx_grouped_gemm_wgrad"):
    _SIGS[_n + "_tiled"] = _SIGS[_n]
# blockwise forward / dgrad for power-of-two scales (on the MX kernel): the same arguments
_SIGS["fp8bw_grouped_gemm_fwd_pow2"] = _SIGS["fp8bw_grouped_gemm_fwd"]
_SIGS["fp8bw_grouped_gemm_dgrad_pow2"] = _SIGS["fp8bw_grouped_gemm_dgrad"]
_SIGS["fp8bw_grouped_gemm_wgrad_pow2"] = _SIGS["fp8bw_grouped_gemm_wgrad"]
# the full-rate FP8 operand feed: the same arguments as the precise entry points
for _n in ("fp8bw_grouped_gemm_fwd_pow2", "fp8bw_grouped_gemm_dgrad_pow2", "fp8bw_grouped_gemm_wgrad_pow2", "mx_grouped_gemm_fwd", "mx_grouped_gemm_dgrad", "mx_grouped_gemm_wgrad", "fp8bw_grouped_gemm_fwd",
           "fp8bw_grouped_gemm_dgrad", "fp8bw_grouped_gemm_wgrad", "mx_grouped_gemm_fwd_tiled",
           "mx_grouped_gemm_dgrad_tiled", "mx_grouped_gemm_wgrad_tiled"):
    _SIGS[_n + "_fp8feed"] = _SIGS[_n]
EXPORTED_SYMBOLS = tuple(_SIGS)


class MxMoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmxmoe (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m precision_moe_expert_mx_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MxMoeError(fn, status, lib().mxmoe_last_error().decode(errors="replace"))


def abi_version() -> int:
    return lib().mxmoe_abi_version()


def mx_colwise_ld_min(M: int, G: int) -> int:
    return lib().mx_colwise_ld_min(int(M), int(G))


def mxmoe_pitch(min_ld: int) -> int:
    """The recommended row pitch >= min_ld for a column-wise output (avoids slow pitches)."""
    return lib().mxmoe_pitch(int(min_ld))


def mxfp4_colwise_ld(M: int, G: Optional[int] = None) -> int:
    """Default leading dimension (elements) of a column-wise MXFP4 output: qT rows hold ld / 2 bytes, so
    the recommended pitch applies to the byte count."""
    need = mx_colwise_ld_min(M, G) if G is not None else 32 * ((int(M) + 31) // 32)
    return 2 * mxmoe_pitch(need // 2)


def mx_colwise_ld(M: int, G: Optional[int] = None) -> int:
    """Default leading dimension of a column-wise MX output of R = M rows: the recommended pitch for G
    groups (routing offsets), or for one group of M rows when G is None (a weight viewed as [G*N, K])."""
    need = mx_colwise_ld_min(M, G) if G is not None else 32 * ((int(M) + 31) // 32)
    return mxmoe_pitch(need)


# ---------------------------------------------------------------- torch plumbing
def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _bf16_bits(x):
    torch = _torch()
    if x.dtype == torch.bfloat16 or x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError(f"expected bfloat16 (or its 16-bit pattern), got {x.dtype}")


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


def _out_dtype(dt: str):
    torch = _torch()
    if dt == "f32":
        return torch.float32, MXMOE_F32
    if dt == "bf16":
        return torch.bfloat16, MXMOE_BF16
    raise ValueError(dt)


def _gemm(name: str, fast: bool):
    """The entry point of a GEMM: the precise feed, or its full-rate FP8 feed (`name`_fp8feed)."""
    return (name + "_fp8feed" if fast else name), getattr(lib(), name + "_fp8feed" if fast else name)


def _call(entry, *args):
    name, f = entry
    return name, f(*args)


# ---------------------------------------------------------------- MX quantisers
def _rowwise_scales_out(R, C, tiled, like):
    """A row-wise copy's scale buffer: [R, C / 32], or [C / 128, R, 4] in the tiled layout."""
    torch = _torch()
    return _empty((C // 128, R, 4) if tiled else (R, C // 32), torch.uint8, like)


def _rowwise(name, tiled, x, q, s, stream):
    torch = _torch()
    x = _bf16_bits(x)
    R, C = x.shape
    q = _empty((R, C), torch.uint8, x) if q is None else q
    s = _rowwise_scales_out(R, C, tiled, x) if s is None else s
    _check(name, getattr(lib(), name)(_ptr(x), R, C, _ptr(q), _ptr(s), _stream_handle(stream)))
    return q, s


def mx_quantize_rowwise(x, q=None, s=None, stream=None) -> Tuple[object, object]:
    """x bf16 [R, C] -> (q uint8 [R, C], s uint8 [R, C/32])."""
    return _rowwise("mx_quantize_rowwise", False, x, q, s, stream)


def mx_quantize_rowwise_tiled(x, q=None, s=None, stream=None) -> Tuple[object, object]:
    """As mx_quantize_rowwise with the scales in the tiled layout: s uint8 [C/128, R, 4] (C % 128 == 0)."""
    return _rowwise("mx_quantize_rowwise_tiled", True, x, q, s, stream)


def _colwise_out(C, ld, tiled, like):
    """A column-wise code buffer: [C, ld] row-major, or [ld / 128, C, 128] in the tiled layout."""
    torch = _torch()
    return _empty((ld // 128, C, 128) if tiled else (C, ld), torch.uint8, like)


def _colwise_scales_out(C, ld, tiled, like):
    """Its scale buffer: [C, ld / 32] row-major, or [ld / 128, C, 4] in the tiled layout."""
    torch = _torch()
    return _empty((ld // 128, C, 4) if tiled else (C, ld // 32), torch.uint8, like)


def _colwise(name, tiled, x, offs, G, ld, qT, sT, stream):
    torch = _torch()
    x = _bf16_bits(x)
    R, C = x.shape
    if offs is not None:
        G = offs.numel() - 1
    if ld is None:
        ld = mx_colwise_ld(R, G if offs is not None else None)
    qT = _colwise_out(C, ld, tiled, x) if qT is None else qT
    sT = _colwise_scales_out(C, ld, tiled, x) if sT is None else sT
    _check(name, getattr(lib(), name)(_ptr(x), R, C, _ptr(offs), G, _ptr(qT), _ptr(sT), ld, _stream_handle(stream)))
    return qT, sT


def mx_quantize_colwise(x, offs=None, G: int = 1, ld: Optional[int] = None, qT=None, sT=None, stream=None):
    """x bf16 [R, C] -> (qT uint8 [C, ld], sT uint8 [C, ld/32]); offs int32 [G+1] device or None."""
    return _colwise("mx_quantize_colwise", False, x, offs, G, ld, qT, sT, stream)


def mx_quantize_colwise_tiled(x, offs=None, G: int = 1, ld: Optional[int] = None, qT=None, sT=None, stream=None):
    """As mx_quantize_colwise in the 128-byte tiled layout: qT uint8 [ld/128, C, 128], sT [ld/128, C, 4]."""
    return _colwise("mx_quantize_colwise_tiled", True, x, offs, G, ld, qT, sT, stream)


def _dual(name, tiled, x, offs, G, ld, row_idx, q, s, qT, sT, stream):
    torch = _torch()
    x = _bf16_bits(x)
    R_src, C = x.shape
    R = row_idx.numel() if row_idx is not None else R_src
    if offs is not None:
        G = offs.numel() - 1
    if ld is None:
        ld = mx_colwise_ld(R, G if offs is not None else None)
    q = _empty((R, C), torch.uint8, x) if q is None else q
    s = _rowwise_scales_out(R, C, tiled, x) if s is None else s
    qT = _colwise_out(C, ld, tiled, x) if qT is None else qT
    sT = _colwise_scales_out(C, ld, tiled, x) if sT is None else sT
    _check(name, getattr(lib(), name)(_ptr(x), R, C, _ptr(row_idx), R_src, _ptr(offs), G, _ptr(q), _ptr(s), _ptr(qT),
                                      _ptr(sT), ld, _stream_handle(stream)))
    return q, s, qT, sT


def mx_quantize_dual(x, offs=None, G: int = 1, ld: Optional[int] = None, row_idx=None, q=None, s=None, qT=None,
                     sT=None, stream=None):
    """Row-wise and column-wise MX layouts from one read of x.

    x bf16 [R_src, C]; row_idx int32 [R] (routed row r reads x[row_idx[r]]) or None (R = R_src).
    Returns (q [R, C], s [R, C/32], qT [C, ld], sT [C, ld/32]), all uint8."""
    return _dual("mx_quantize_dual", False, x, offs, G, ld, row_idx, q, s, qT, sT, stream)


def mx_quantize_dual_tiled(x, offs=None, G: int = 1, ld: Optional[int] = None, row_idx=None, q=None, s=None,
                           qT=None, sT=None, stream=None):
    """As mx_quantize_dual in the 128-byte tiled layouts: qT [ld/128, C, 128], sT [ld/128, C, 4] and
    s [C/128, R, 4] (C % 128 == 0)."""
    return _dual("mx_quantize_dual_tiled", True, x, offs, G, ld, row_idx, q, s, qT, sT, stream)


# ---------------------------------------------------------------- MX grouped GEMMs
def _fwd(name, qx, sx, qw, sw, offs, N, out_dtype, y, stream, fast):
    M, K = qx.shape
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    y = _empty((M, N), tdt, qx) if y is None else y
    _check(*_call(_gemm(name, fast), _ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(offs), G, M, N, K, _ptr(y), cdt,
                  _stream_handle(stream)))
    return y


def mx_grouped_gemm_fwd(qx, sx, qw, sw, offs, N: int, out_dtype: str = "f32", y=None, stream=None, fast: bool = False):
    """Y [M, N] = per-expert X_g W_g^T from row-wise MX operands (qw: [G*N, K])."""
    return _fwd("mx_grouped_gemm_fwd", qx, sx, qw, sw, offs, N, out_dtype, y, stream, fast)


def mx_grouped_gemm_fwd_tiled(qx, sx, qw, sw, offs, N: int, out_dtype: str = "f32", y=None, stream=None,
                              fast: bool = False):
    """As mx_grouped_gemm_fwd with the scales in the tiled layout (sx [K/128, M, 4], sw [K/128, G*N, 4])."""
    return _fwd("mx_grouped_gemm_fwd_tiled", qx, sx, qw, sw, offs, N, out_dtype, y, stream, fast)


def _swiglu(name, tiled, qx, sx, qw, sw, offs, N, y, qh, sh, h, with_h, colwise, ldh, qhT, shT, stream):
    torch = _torch()
    M, K = qx.shape
    G = offs.numel() - 1
    H = N // 2
    y = _empty((M, N), torch.bfloat16, qx) if y is None else y
    qh = _empty((M, H), torch.uint8, qx) if qh is None else qh
    sh = _rowwise_scales_out(M, H, tiled, qx) if sh is None else sh
    if with_h and h is None:
        h = _empty((M, H), torch.float32, qx)
    if colwise or tiled or qhT is not None:
        if qhT is not None:
            ldh = qhT.shape[0] * 128 if tiled else qhT.shape[1]
        elif ldh is None:
            ldh = mx_colwise_ld(M, G)
        qhT = _colwise_out(H, ldh, tiled, qx) if qhT is None else qhT
        shT = _colwise_scales_out(H, ldh, tiled, qx) if shT is None else shT
    _check(name, getattr(lib(), name)(
        _ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(offs), G, M, N, K, _ptr(y), _ptr(qh), _ptr(sh), _ptr(h),
        _ptr(qhT), _ptr(shT), int(ldh or 0), _stream_handle(stream)))
    out = (y, qh, sh) + ((qhT, shT) if qhT is not None else ())
    return out if h is None else out + (h,)


def mx_grouped_gemm_fwd_swiglu(qx, sx, qw, sw, offs, N: int, y=None, qh=None, sh=None, h=None,
                               with_h: bool = False, colwise: bool = False, ldh: Optional[int] = None, qhT=None,
                               shT=None, stream=None):
    """Forward of the gate+up GEMM (W rows: gate then up of each expert, N = 2H) with SwiGLU and the
    MX quantisation of H in the epilogue.  Returns (y bf16 [M, N], qh [M, H], sh [M, H/32]); with
    colwise (or qhT given) also H column-wise (qhT [H, ldh], shT [H, ldh/32], ldh by default the
    recommended pitch for the routing offsets); with with_h (or h given) H in fp32 [M, H] last."""
    return _swiglu("mx_grouped_gemm_fwd_swiglu", False, qx, sx, qw, sw, offs, N, y, qh, sh, h, with_h, colwise, ldh,
                   qhT, shT, stream)


def mx_grouped_gemm_fwd_swiglu_tiled(qx, sx, qw, sw, offs, N: int, y=None, qh=None, sh=None, h=None,
                                     with_h: bool = False, ldh: Optional[int] = None, qhT=None, shT=None,
                                     stream=None):
    """As mx_grouped_gemm_fwd_swiglu in the 128-byte tiled layouts: sx [K/128, M, 4] and sw [K/128, G*N, 4]
    in; sh [H/128, M, 4], qhT [ldh/128, H, 128], shT [ldh/128, H, 4] out (H always column-wise too).
    Returns (y, qh, sh, qhT, shT[, h])."""
    return _swiglu("mx_grouped_gemm_fwd_swiglu_tiled", True, qx, sx, qw, sw, offs, N, y, qh, sh, h, with_h, True,
                   ldh, qhT, shT, stream)


def mx_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs, K: int, out_dtype: str = "f32", dx=None, stream=None, fast: bool = False):
    """dX [M, K] = per-expert dY_g W_g from row-wise dY and column-wise W ([K, ldw])."""
    return _dgrad("mx_grouped_gemm_dgrad", qwT.shape[1], qdy, sdy, qwT, swT, offs, K, out_dtype, dx, stream, fast)


def mx_grouped_gemm_dgrad_tiled(qdy, sdy, qwT, swT, offs, K: int, out_dtype: str = "f32", dx=None, stream=None,
                                fast: bool = False):
    """As mx_grouped_gemm_dgrad in the 128-byte tiled layouts: sdy [N/128, M, 4], qwT [ldw/128, K, 128],
    swT [ldw/128, K, 4]."""
    return _dgrad("mx_grouped_gemm_dgrad_tiled", qwT.shape[0] * 128, qdy, sdy, qwT, swT, offs, K, out_dtype, dx,
                  stream, fast)


def _dgrad(name, ldw, qdy, sdy, qwT, swT, offs, K, out_dtype, dx, stream, fast):
    M, N = qdy.shape
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    dx = _empty((M, K), tdt, qdy) if dx is None else dx
    _check(*_call(_gemm(name, fast), _ptr(qdy), _ptr(sdy), _ptr(qwT), _ptr(swT), ldw, _ptr(offs), G, M, N, K,
                  _ptr(dx), cdt, _stream_handle(stream)))
    return dx


def mx_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, M: int, out_dtype: str = "f32", dw=None, stream=None, fast: bool = False):
    """dW [G, N, K] = per-expert dY_g^T X_g from column-wise dY ([N, ld]) and X ([K, ld])."""
    N, ld = qdyT.shape
    return _wgrad("mx_grouped_gemm_wgrad", N, ld, qxT.shape[0], qdyT, sdyT, qxT, sxT, offs, M, out_dtype, dw, stream,
                  fast)


def mx_grouped_gemm_wgrad_tiled(qdyT, sdyT, qxT, sxT, offs, M: int, out_dtype: str = "f32", dw=None, stream=None,
                                fast: bool = False):
    """As mx_grouped_gemm_wgrad with qdyT, sdyT / qxT, sxT in the 128-byte tiled layout
    ([ld/128, N, 128], [ld/128, N, 4] / [ld/128, K, 128], [ld/128, K, 4])."""
    return _wgrad("mx_grouped_gemm_wgrad_tiled", qdyT.shape[1], qdyT.shape[0] * 128, qxT.shape[1], qdyT, sdyT, qxT,
                  sxT, offs, M, out_dtype, dw, stream, fast)


def _wgrad(name, N, ld, K, qdyT, sdyT, qxT, sxT, offs, M, out_dtype, dw, stream, fast):
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    dw = _empty((G, N, K), tdt, qdyT) if dw is None else dw
    _check(*_call(_gemm(name, fast), _ptr(qdyT), _ptr(sdyT), _ptr(qxT), _ptr(sxT), ld, _ptr(offs), G, M, N, K,
                  _ptr(dw), cdt, _stream_handle(stream)))
    return dw


# ---------------------------------------------------------------- MXFP4
def mxfp4_quantize_rowwise(x, q=None, s=None, stream=None):
    """x bf16 [R, C] -> (q uint8 [R, C/2] packed E2M1, s uint8 [R, C/32])."""
    torch = _torch()
    x = _bf16_bits(x)
    R, C = x.shape
    q = _empty((R, C // 2), torch.uint8, x) if q is None else q
    s = _empty((R, C // 32), torch.uint8, x) if s is None else s
    _check("mxfp4_quantize_rowwise", lib().mxfp4_quantize_rowwise(_ptr(x), R, C, _ptr(q), _ptr(s),
                                                                  _stream_handle(stream)))
    return q, s


def mxfp4_quantize_colwise(x, offs=None, G: int = 1, ld: Optional[int] = None, qT=None, sT=None, stream=None):
    """x bf16 [R, C] -> (qT uint8 [C, ld/2] packed E2M1, sT uint8 [C, ld/32])."""
    torch = _torch()
    x = _bf16_bits(x)
    R, C = x.shape
    if offs is not None:
        G = offs.numel() - 1
    if ld is None:
        ld = mxfp4_colwise_ld(R, G if offs is not None else None)
    qT = _empty((C, ld // 2), torch.uint8, x) if qT is None else qT
    sT = _empty((C, ld // 32), torch.uint8, x) if sT is None else sT
    _check("mxfp4_quantize_colwise", lib().mxfp4_quantize_colwise(_ptr(x), R, C, _ptr(offs), G, _ptr(qT), _ptr(sT),
                                                                  ld, _stream_handle(stream)))
    return qT, sT


def mxfp4_grouped_gemm_fwd(qx, sx, qw, sw, offs, N: int, out_dtype: str = "f32", y=None, stream=None):
    """Y [M, N] from row-wise MXFP4 X (qx [M, K/2]) and W (qw [G*N, K/2])."""
    M, K = qx.shape[0], 2 * qx.shape[1]
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    y = _empty((M, N), tdt, qx) if y is None else y
    _check("mxfp4_grouped_gemm_fwd", lib().mxfp4_grouped_gemm_fwd(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(offs),
                                                                  G, M, N, K, _ptr(y), cdt, _stream_handle(stream)))
    return y


def mxfp4_grouped_gemm_dgrad(qdy, sdy, qwT, swT, offs, K: int, out_dtype: str = "f32", dx=None, stream=None):
    """dX [M, K] from row-wise MXFP4 dY (qdy [M, N/2]) and column-wise W (qwT [K, ldw/2])."""
    M, N = qdy.shape[0], 2 * qdy.shape[1]
    ldw = 2 * qwT.shape[1]
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    dx = _empty((M, K), tdt, qdy) if dx is None else dx
    _check("mxfp4_grouped_gemm_dgrad", lib().mxfp4_grouped_gemm_dgrad(_ptr(qdy), _ptr(sdy), _ptr(qwT), _ptr(swT), ldw,
                                                                      _ptr(offs), G, M, N, K, _ptr(dx), cdt,
                                                                      _stream_handle(stream)))
    return dx


def mxfp4_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, M: int, out_dtype: str = "f32", dw=None, stream=None):
    """dW [G, N, K] from column-wise MXFP4 dY (qdyT [N, ld/2]) and X (qxT [K, ld/2])."""
    N, ld = qdyT.shape[0], 2 * qdyT.shape[1]
    K = qxT.shape[0]
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    dw = _empty((G, N, K), tdt, qdyT) if dw is None else dw
    _check("mxfp4_grouped_gemm_wgrad", lib().mxfp4_grouped_gemm_wgrad(_ptr(qdyT), _ptr(sdyT), _ptr(qxT), _ptr(sxT), ld,
                                                                      _ptr(offs), G, M, N, K, _ptr(dw), cdt,
                                                                      _stream_handle(stream)))
    return dw


# ---------------------------------------------------------------- blockwise FP8
def fp8bw_quantize_act_1x128(x, q=None, s=None, stream=None, pow2: bool = False):
    """x bf16 [R, C] -> (q [R, C], s f32 [R, C/128]); pow2 selects the power-of-two scale mode."""
    torch = _torch()
    x = _bf16_bits(x)
    R, C = x.shape
    q = _empty((R, C), torch.uint8, x) if q is None else q
    s = _empty((R, C // 128), torch.float32, x) if s is None else s
    fn = "fp8bw_quantize_act_1x128" + ("_pow2" if pow2 else "")
    _check(fn, getattr(lib(), fn)(_ptr(x), R, C, _ptr(q), _ptr(s), _stream_handle(stream)))
    return q, s


def fp8bw_quantize_weight_128x128(w, q=None, s=None, qT=None, transposed: bool = False, stream=None,
                                  pow2: bool = False):
    """w bf16 [R, C] -> (q [R, C], s f32 [R/128, C/128]) or, with transposed=True (or qT given),
    (q, s, qT [C, R]) where qT is the dgrad operand; pow2 selects the power-of-two scale mode."""
    torch = _torch()
    w = _bf16_bits(w)
    R, C = w.shape
    q = _empty((R, C), torch.uint8, w) if q is None else q
    s = _empty((R // 128, C // 128), torch.float32, w) if s is None else s
    if transposed and qT is None:
        qT = _empty((C, R), torch.uint8, w)
    fn = "fp8bw_quantize_weight_128x128" + ("_pow2" if pow2 else "")
    _check(fn, getattr(lib(), fn)(_ptr(w), R, C, _ptr(q), _ptr(s), _ptr(qT), _stream_handle(stream)))
    return (q, s) if qT is None else (q, s, qT)


def _bw_fwd(name, qx, sx, qw, sw, offs, N, out_dtype, y, stream, fast):
    M, K = qx.shape
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    y = _empty((M, N), tdt, qx) if y is None else y
    _check(*_call(_gemm(name, fast), _ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(offs), G, M, N, K, _ptr(y), cdt,
                  _stream_handle(stream)))
    return y


def _bw_dgrad(name, qdy, sdy, qwT, sw, offs, K, out_dtype, dx, stream, fast):
    M, N = qdy.shape
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    dx = _empty((M, K), tdt, qdy) if dx is None else dx
    _check(*_call(_gemm(name, fast), _ptr(qdy), _ptr(sdy), _ptr(qwT), _ptr(sw), _ptr(offs), G, M, N, K, _ptr(dx),
                  cdt, _stream_handle(stream)))
    return dx


def fp8bw_grouped_gemm_fwd(qx, sx, qw, sw, offs, N: int, out_dtype: str = "f32", y=None, stream=None, fast: bool = False):
    """Y [M, N] from blockwise X (1x128 tiles) and W (128x128 blocks), promoted per 128-slice."""
    return _bw_fwd("fp8bw_grouped_gemm_fwd", qx, sx, qw, sw, offs, N, out_dtype, y, stream, fast)


def fp8bw_grouped_gemm_dgrad(qdy, sdy, qwT, sw, offs, K: int, out_dtype: str = "f32", dx=None, stream=None,
                             fast: bool = False):
    """dX [M, K] from blockwise dY (1x128 along N) and the transposed weight copy qwT [K, G*N]."""
    return _bw_dgrad("fp8bw_grouped_gemm_dgrad", qdy, sdy, qwT, sw, offs, K, out_dtype, dx, stream, fast)


def fp8bw_grouped_gemm_fwd_pow2(qx, sx, qw, sw, offs, N: int, out_dtype: str = "f32", y=None, stream=None,
                                fast: bool = False):
    """fp8bw_grouped_gemm_fwd for power-of-two scales (the _pow2 quantisers' output), on the MX kernel."""
    return _bw_fwd("fp8bw_grouped_gemm_fwd_pow2", qx, sx, qw, sw, offs, N, out_dtype, y, stream, fast)


def fp8bw_grouped_gemm_dgrad_pow2(qdy, sdy, qwT, sw, offs, K: int, out_dtype: str = "f32", dx=None, stream=None,
                                  fast: bool = False):
    """fp8bw_grouped_gemm_dgrad for power-of-two scales (the _pow2 quantisers' output), on the MX kernel."""
    return _bw_dgrad("fp8bw_grouped_gemm_dgrad_pow2", qdy, sdy, qwT, sw, offs, K, out_dtype, dx, stream, fast)


def fp8bw_colwise_ld_min(M: int, G: int) -> int:
    """Smallest leading dimension of the column-wise blockwise layout (host arithmetic)."""
    return int(lib().fp8bw_colwise_ld_min(M, G))


def fp8bw_quantize_colwise_128(x, offs=None, G: int = 1, ld: Optional[int] = None, qT=None, sT=None, stream=None,
                               pow2: bool = False):
    """x bf16 [R, C] -> (qT uint8 [C, ld], sT float32 [C, ld/128]): 128-row blocks restarting per group;
    pow2 selects the power-of-two scale mode."""
    torch = _torch()
    x = _bf16_bits(x)
    R, C = x.shape
    if offs is not None:
        G = offs.numel() - 1
    if ld is None:
        ld = fp8bw_colwise_ld_min(R, G) if offs is not None else 128 * ((R + 127) // 128)
    qT = _empty((C, ld), torch.uint8, x) if qT is None else qT
    sT = _empty((C, ld // 128), torch.float32, x) if sT is None else sT
    fn = "fp8bw_quantize_colwise_128" + ("_pow2" if pow2 else "")
    _check(fn, getattr(lib(), fn)(_ptr(x), R, C, _ptr(offs), G, _ptr(qT), _ptr(sT), ld, _stream_handle(stream)))
    return qT, sT


def _bw_wgrad(name, qdyT, sdyT, qxT, sxT, offs, M, out_dtype, dw, stream, fast):
    N, ld = qdyT.shape
    K = qxT.shape[0]
    G = offs.numel() - 1
    tdt, cdt = _out_dtype(out_dtype)
    dw = _empty((G, N, K), tdt, qdyT) if dw is None else dw
    _check(*_call(_gemm(name, fast), _ptr(qdyT), _ptr(sdyT), _ptr(qxT), _ptr(sxT), ld, _ptr(offs), G, M, N, K,
                  _ptr(dw), cdt, _stream_handle(stream)))
    return dw


def fp8bw_grouped_gemm_wgrad(qdyT, sdyT, qxT, sxT, offs, M: int, out_dtype: str = "f32", dw=None, stream=None,
                             fast: bool = False):
    """dW [G, N, K] from the column-wise blockwise copies of dY [N, ld] and X [K, ld]."""
    return _bw_wgrad("fp8bw_grouped_gemm_wgrad", qdyT, sdyT, qxT, sxT, offs, M, out_dtype, dw, stream, fast)


def fp8bw_grouped_gemm_wgrad_pow2(qdyT, sdyT, qxT, sxT, offs, M: int, out_dtype: str = "f32", dw=None, stream=None,
                                  fast: bool = False):
    """fp8bw_grouped_gemm_wgrad for power-of-two scales (the _pow2 quantisers' output), on the MX kernel."""
    return _bw_wgrad("fp8bw_grouped_gemm_wgrad_pow2", qdyT, sdyT, qxT, sxT, offs, M, out_dtype, dw, stream, fast)


def mxmoe_check_offsets(offs, M: int, stream=None) -> None:
    G = offs.numel() - 1
    _check("mxmoe_check_offsets", lib().mxmoe_check_offsets(_ptr(offs), G, M, _stream_handle(stream)))
