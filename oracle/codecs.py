"""Element and scale codecs (oracle; test infrastructure only).

E4M3 and E8M0 as defined by the OCP Microscaling Formats (MX) v1.0
specification, which the pages name only as "MXFP8" (opensourcebeat.com,
FAQ "What is MXFP8?") and "E4M3" (aifind.ru DeepSeek-V3 article, section on
concerns about FP8 range).  The E4M3 variant is OCP "FN": exponent bias 7,
largest finite value 448 (code 0x7E), codes 0x7F / 0xFF are NaN, no infinity.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Value of E4M3-FN codes.

    sign s, exponent field E (4 bits), mantissa m (3 bits):
      E == 0 : (-1)^s * m * 2^-9          (subnormal; 0x00 / 0x80 are +-0)
      E >  0 : (-1)^s * (1 + m/8) * 2^(E-7)
      s.1111.111 : NaN
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# the 127 non-negative finite codes 0x00..0x7E decode to strictly increasing values
_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(y) -> np.ndarray:
    """Round finite reals to E4M3-FN: nearest, ties to even, saturating at +-448.

    Reading (pages silent): round-to-nearest-even, overflow saturates to the
    largest finite magnitude (E4M3-FN has no infinity), the sign is kept so a
    negative value that rounds to zero encodes as 0x80 (-0).

    The representable magnitudes below 2^(e+1) with e >= -6 are the multiples
    of 2^(e-3), so |y| is divided by that quantum (exact: a power of two),
    rounded half-to-even (np.rint), and multiplied back.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3_encode: non-finite input is outside the contract")
    a = np.abs(y)
    _, ex = np.frexp(a)                      # a = f * 2^ex with f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # floor(log2 a), clamped at the subnormal binade
    quantum = np.ldexp(1.0, e - 3)
    r = np.rint(a / quantum) * quantum
    r = np.minimum(r, E4M3_MAX)
    code = np.searchsorted(_POS, r)
    if not np.array_equal(_POS[np.minimum(code, 0x7E)], r):
        raise AssertionError("e4m3_encode: rounded value not representable")
    sign = np.where(np.signbit(y), 0x80, 0)
    return (code | sign).astype(np.uint8)


def e4m3_encode_bruteforce(y) -> np.ndarray:
    """Independent encoder for pinning `e4m3_encode` on small inputs.

    Picks, among all 127 finite magnitudes, the one nearest to |y| (|y| first
    clamped to 448); on a tie it takes the code with an even mantissa field.
    Slow (O(127) per element): used only by tests.
    """
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    out = np.empty(y.shape, dtype=np.uint8)
    for i, v in enumerate(y):
        a = min(abs(float(v)), E4M3_MAX)
        d = np.abs(_POS - a)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            even = [c for c in best if (c & 1) == 0]
            best = even
        c = int(best[0])
        out[i] = c | (0x80 if np.signbit(v) else 0)
    return out


def e8m0_decode(b) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(b - 127) for b in [0, 254]; 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, (b - 127).astype(np.int64)))


# ----------------------------------------------------------------------------------------- E2M1 (FP4)
# OCP MX v1.0, FP4 element "E2M1": sign, 2 exponent bits (bias 1), 1 mantissa bit; no infinity or NaN;
# largest magnitude 6.  The pages only announce a 4-bit format as the next step (iitak.ru article,
# closing section); MXFP4 is that format on the MX scale of E8M0 per 32 elements.
E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """Value of E2M1 codes (0..15):
      E == 0 : (-1)^s * m * 0.5             (0x0 / 0x8 are +-0, 0x1 = 0.5)
      E >  0 : (-1)^s * (1 + m/2) * 2^(E-1)  (1, 1.5, 2, 3, 4, 6)
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


_POS4 = e2m1_decode(np.arange(8))


def e2m1_encode(y) -> np.ndarray:
    """Round finite reals to E2M1: nearest, ties to even, saturating at +-6 (same readings as E4M3:
    the pages are silent).  Below 2^(e+1) with e >= 0 the representable magnitudes are the multiples
    of 2^(e-1), so |y| is divided by that quantum, rounded half-to-even and multiplied back."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("e2m1_encode: non-finite input is outside the contract")
    a = np.abs(y)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, 0)
    quantum = np.ldexp(1.0, e - 1)
    r = np.minimum(np.rint(a / quantum) * quantum, E2M1_MAX)
    code = np.searchsorted(_POS4, r)
    if not np.array_equal(_POS4[np.minimum(code, 7)], r):
        raise AssertionError("e2m1_encode: rounded value not representable")
    sign = np.where(np.signbit(y), 0x8, 0)
    return (code | sign).astype(np.uint8)


def e2m1_encode_bruteforce(y) -> np.ndarray:
    """Independent encoder: the nearest of the 8 magnitudes (|y| clamped to 6), ties to the code with
    an even mantissa bit."""
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    out = np.empty(y.shape, dtype=np.uint8)
    for i, v in enumerate(y):
        a = min(abs(float(v)), E2M1_MAX)
        d = np.abs(_POS4 - a)
        best = [c for c in np.flatnonzero(d == d.min())]
        if len(best) > 1:
            best = [c for c in best if (c & 1) == 0]
        out[i] = int(best[0]) | (0x8 if np.signbit(v) else 0)
    return out


def fp4_pack(codes) -> np.ndarray:
    """Pack E2M1 codes along the last axis, two per byte: element 2i in the low nibble, 2i+1 in the
    high nibble (a layout choice: OCP MX leaves packing to the implementation)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def fp4_unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
