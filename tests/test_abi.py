"""The C-ABI library loads, exports every entry point declared in include/mxmoe.h, and rejects bad
arguments on the host (no GPU needed: validation happens before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")


def _lib():
    import precision_moe_expert_mx_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmxmoe.so not built (run __graft_entry__.build())")
    return m, m.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declarations_match_binding():
    import precision_moe_expert_mx_amd as m
    assert _declared() == sorted(m.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    m, L = _lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert m.abi_version() == 5


def test_host_helpers():
    m, L = _lib()
    assert [m.mx_colwise_ld_min(M, G) for M, G in ((1024, 4), (49152, 64), (65536, 8), (32768, 16))] == \
        [1152, 51136, 65792, 33280]
    assert m.mx_colwise_ld_min(-1, 4) == -1 and m.mx_colwise_ld_min(10, 0) == -1
    assert [m.fp8bw_colwise_ld_min(M, G) for M, G in ((1024, 4), (49152, 64), (65536, 8))] == \
        [1536, 57344, 66560]
    assert m.fp8bw_colwise_ld_min(-1, 4) == -1 and m.fp8bw_colwise_ld_min(10, 0) == -1


def test_recommended_pitch():
    m, L = _lib()
    slow = {(1 << p) + (1 << (p - k)) for p in range(7, 40) for k in (7, 8, 9) if p >= k}
    # the expert-shard minimum 2^16 + 2^8 and the slow weight pitch 2^15 + 2^7 move up by 1 KiB
    assert m.mxmoe_pitch(65792) == 65792 + 1024
    assert m.mxmoe_pitch(32896) == 32896 + 1024
    # the other configs' minima and powers of two are kept, rounded up to a multiple of 128
    for ld in (1152, 33280, 32768, 57344, 131072, 180224, 65536):
        assert m.mxmoe_pitch(ld) == ld
    assert m.mxmoe_pitch(51136) == 51200 and m.mxmoe_pitch(1088) == 1152
    assert m.mxmoe_pitch(-1) == -1 and m.mxmoe_pitch(0) == 0
    assert m.mxmoe_pitch((1 << 62) + (1 << 54)) >= (1 << 62) + (1 << 54)   # no overflow near the top
    rng = np.random.default_rng(5)
    cands = sorted(slow) + [int(v) for v in rng.integers(0, 1 << 24, 2000) * 32]
    for ld in cands:
        got = m.mxmoe_pitch(ld)
        want = (ld + 127) // 128 * 128
        while want in slow:
            want += 1024
        assert got == want, (ld, got, want)
    assert m.mx_colwise_ld(65536, 8) == 66816 and m.mx_colwise_ld(49152, 64) == 51200
    assert m.mx_colwise_ld(32768) == 32768
    # E2M1 rows hold ld / 2 bytes: the shard's 65792 / 2 = 2^15 + 2^7 bytes is a slow pitch
    assert m.mxfp4_colwise_ld(65536, 8) == 2 * (32896 + 1024) and m.mxfp4_colwise_ld(49152, 64) == 51200


A16 = 0x10000      # fake, 16-byte aligned device addresses: never dereferenced on error paths
A16b = 0x20000
BAD = 0x10001


def _status(L, fn, *args):
    st = getattr(L, fn)(*args)
    return st, L.mxmoe_last_error().decode()


def test_quantiser_argument_errors():
    _, L = _lib()
    st, msg = _status(L, "mx_quantize_rowwise", A16, 4, 33, A16, A16, None)
    assert st == 2 and "32" in msg
    assert _status(L, "mx_quantize_rowwise", A16, -1, 32, A16, A16, None)[0] == 2
    assert _status(L, "mx_quantize_rowwise", None, 4, 64, A16, A16, None)[0] == 1
    assert _status(L, "mx_quantize_rowwise", BAD, 4, 64, A16, A16, None)[0] == 3
    assert _status(L, "mx_quantize_rowwise", A16, 0, 64, None, None, None) == (0, "")   # empty: no-op
    # column-wise: ld too small / not a multiple of 32 / G out of range
    assert _status(L, "mx_quantize_colwise", A16, 100, 64, A16, 4, A16, A16, 96, None)[0] == 2
    assert _status(L, "mx_quantize_colwise", A16, 100, 64, A16, 4, A16, A16, 250, None)[0] == 3
    assert _status(L, "mx_quantize_colwise", A16, 100, 64, A16, 0, A16, A16, 256, None)[0] == 2
    assert _status(L, "mx_quantize_colwise", A16, 100, 64, None, 0, A16, A16, 96, None)[0] == 2    # needs 128
    assert _status(L, "mx_quantize_colwise", A16, 100, 64, None, 0, None, A16, 128, None)[0] == 1
    # blockwise
    assert _status(L, "fp8bw_quantize_act_1x128", A16, 4, 96, A16, A16, None)[0] == 2
    assert _status(L, "fp8bw_quantize_weight_128x128", A16, 100, 128, A16, A16, None, None)[0] == 2
    assert _status(L, "fp8bw_quantize_weight_128x128", A16, 128, 128, A16, A16, BAD, None)[0] == 3
    # blockwise column-wise: C % 128, ld % 128, ld too small
    assert _status(L, "fp8bw_quantize_colwise_128", A16, 100, 96, A16, 4, A16, A16, 640, None)[0] == 2
    assert _status(L, "fp8bw_quantize_colwise_128", A16, 100, 128, A16, 4, A16, A16, 600, None)[0] == 3
    assert _status(L, "fp8bw_quantize_colwise_128", A16, 100, 128, A16, 4, A16, A16, 512, None)[0] == 2
    assert _status(L, "fp8bw_quantize_colwise_128", A16, 200, 128, None, 0, A16, A16, 128, None)[0] == 2   # one group
    # the power-of-two mode validates the same way
    assert _status(L, "fp8bw_quantize_act_1x128_pow2", A16, 4, 96, A16, A16, None)[0] == 2
    assert _status(L, "fp8bw_quantize_weight_128x128_pow2", A16, 128, 128, A16, A16, BAD, None)[0] == 3
    assert _status(L, "fp8bw_quantize_colwise_128_pow2", A16, 100, 128, A16, 4, A16, A16, 512, None)[0] == 2


def test_gemm_argument_errors():
    _, L = _lib()
    ok_args = (A16, A16, A16b, A16b, A16, 4, 1024, 512, 256, A16, 0, None)
    # N not a multiple of 128
    a = list(ok_args); a[7] = 500
    assert _status(L, "mx_grouped_gemm_fwd", *a)[0] == 2
    a = list(ok_args); a[5] = 0
    assert _status(L, "mx_grouped_gemm_fwd", *a)[0] == 2           # G < 1
    a = list(ok_args); a[10] = 7
    assert _status(L, "mx_grouped_gemm_fwd", *a)[0] == 4           # dtype
    a = list(ok_args); a[4] = None
    assert _status(L, "mx_grouped_gemm_fwd", *a)[0] == 1           # offsets
    a = list(ok_args); a[9] = BAD
    assert _status(L, "mx_grouped_gemm_fwd", *a)[0] == 3           # output alignment
    a = list(ok_args); a[6] = 0
    assert _status(L, "mx_grouped_gemm_fwd", *a) == (0, "")       # M == 0: no-op
    # dgrad: ldw < G*N
    st, msg = _status(L, "mx_grouped_gemm_dgrad", A16, A16, A16b, A16b, 1024, A16, 4, 1024, 512, 256, A16, 0, None)
    assert st == 2 and "ldw" in msg
    # wgrad: ld < mx_colwise_ld_min
    st, msg = _status(L, "mx_grouped_gemm_wgrad", A16, A16, A16b, A16b, 1024, A16, 4, 1024, 512, 256, A16, 0, None)
    assert st == 2 and "ld" in msg
    # operand rows too long for the 32-bit offsets of a 256-row tile (K = 2^25 bytes per row)
    a = list(ok_args); a[8] = 1 << 25
    st, msg = _status(L, "mx_grouped_gemm_fwd", *a)
    assert st == 2 and "stride" in msg
    st, msg = _status(L, "mx_grouped_gemm_wgrad", A16, A16, A16b, A16b, 1 << 25, A16, 4, 1024, 512, 256, A16, 0, None)
    assert st == 2 and "stride" in msg
    # blockwise
    a = list(ok_args); a[8] = 200
    assert _status(L, "fp8bw_grouped_gemm_fwd", *a)[0] == 2
    assert _status(L, "mxmoe_check_offsets", A16, 0, 10, None)[0] == 2
    # blockwise wgrad: ld not a multiple of 128 / below fp8bw_colwise_ld_min
    st, msg = _status(L, "fp8bw_grouped_gemm_wgrad", A16, A16, A16b, A16b, 1184, A16, 4, 1024, 512, 256, A16, 0, None)
    assert st == 2 and "ld" in msg
    assert _status(L, "fp8bw_grouped_gemm_wgrad", A16, A16, A16b, A16b, 1408, A16, 4, 1024, 512, 256, A16, 0,
                   None)[0] == 2


def test_fp8_feed_entry_points_validate_like_the_precise_ones():
    """The full-rate FP8 feed has entry points of its own (same arguments); the output dtype argument
    takes exactly MXMOE_F32 or MXMOE_BF16 (no feed bits)."""
    _, L = _lib()
    ok_args = (A16, A16, A16b, A16b, A16, 4, 1024, 512, 256, A16, 0, None)
    for fn in ("mx_grouped_gemm_fwd", "mx_grouped_gemm_fwd_fp8feed", "fp8bw_grouped_gemm_fwd",
               "fp8bw_grouped_gemm_fwd_fp8feed"):
        for dt in (0x100, 0x101, 2, -1):
            a = list(ok_args); a[10] = dt
            st, msg = _status(L, fn, *a)
            assert st == 4 and fn in msg, (fn, dt, msg)
        a = list(ok_args); a[7] = 500
        assert _status(L, fn, *a)[0] == 2
        a = list(ok_args); a[6] = 0
        assert _status(L, fn, *a) == (0, "")
    for fn in ("mx_grouped_gemm_dgrad_fp8feed", "mx_grouped_gemm_wgrad_fp8feed"):
        st, msg = _status(L, fn, A16, A16, A16b, A16b, 1024, A16, 4, 1024, 512, 256, A16, 0, None)
        assert st == 2 and fn in msg
    st, msg = _status(L, "fp8bw_grouped_gemm_wgrad_fp8feed", A16, A16, A16b, A16b, 1184, A16, 4, 1024, 512, 256, A16,
                      0, None)
    assert st == 2 and "fp8feed" in msg
    a = list(ok_args); a[8] = 200
    assert _status(L, "fp8bw_grouped_gemm_dgrad_fp8feed", *a)[0] == 2


def test_tiled_entry_points_need_a_pitch_multiple_of_128():
    """The 128-byte tiled column-wise layout: the same validation as the row-major entry points plus
    ld % 128 == 0 (quantisers: MXMOE_ERR_ALIGN; GEMMs: MXMOE_ERR_SHAPE); the gated forward's tiled
    variant always writes H column-wise."""
    _, L = _lib()
    # R = 1000 rows in 4 groups: minimum ld 1120; 1184 is a multiple of 32 but not of 128
    for fn, args in (("mx_quantize_colwise_tiled", (A16, 1000, 64, A16, 4, A16, A16, 1184, None)),
                     ("mx_quantize_dual_tiled", (A16, 1000, 64, None, 0, A16, 4, A16, A16, A16b, A16b, 1184, None))):
        st, msg = _status(L, fn, *args)
        assert st == 3 and fn in msg and "128" in msg, (fn, st, msg)
    assert _status(L, "mx_quantize_colwise_tiled", A16, 100, 64, A16, 4, A16, A16, 96, None)[0] == 3
    assert _status(L, "mx_quantize_colwise_tiled", A16, 1000, 64, A16, 4, A16, A16, 1024, None)[0] == 2   # < 1120
    assert _status(L, "mx_quantize_colwise_tiled", A16, 100, 64, A16, 4, None, A16, 256, None)[0] == 1
    for fn in ("mx_grouped_gemm_dgrad_tiled", "mx_grouped_gemm_dgrad_tiled_fp8feed"):
        # G * N = 2048: ldw 2080 is a multiple of 32, not of 128
        st, msg = _status(L, fn, A16, A16, A16b, A16b, 2080, A16, 4, 1024, 512, 256, A16, 0, None)
        assert st == 2 and fn in msg and "128" in msg, (fn, msg)
    for fn in ("mx_grouped_gemm_wgrad_tiled", "mx_grouped_gemm_wgrad_tiled_fp8feed"):
        # mx_colwise_ld_min(1024, 4) = 1152; 1184 is above it but not a multiple of 128
        st, msg = _status(L, fn, A16, A16, A16b, A16b, 1184, A16, 4, 1024, 512, 256, A16, 0, None)
        assert st == 2 and fn in msg and "128" in msg, (fn, msg)
        assert _status(L, fn, A16, A16, A16b, A16b, 1024, A16, 4, 1024, 512, 256, A16, 0, None)[0] == 2
    sw = (A16, A16, A16b, A16b, A16, 4, 1024, 512, 256, A16, A16, A16)
    st, msg = _status(L, "mx_grouped_gemm_fwd_swiglu_tiled", *sw, None, None, None, 1152, None)
    assert st == 1 and "qhT" in msg
    st, msg = _status(L, "mx_grouped_gemm_fwd_swiglu_tiled", *sw, None, A16b, A16b, 1184, None)
    assert st == 2 and "128" in msg


def test_tiled_row_wise_scales_need_whole_128_column_slices():
    """Tiled row-wise scales ([C/128][R][4]): the row-wise and dual tiled quantisers refuse C % 128 != 0
    (MXMOE_ERR_SHAPE) where their row-major namesakes accept any C % 32 == 0; the tiled forward GEMM
    validates as mx_grouped_gemm_fwd."""
    _, L = _lib()
    st, msg = _status(L, "mx_quantize_rowwise_tiled", A16, 100, 96, A16, A16, None)
    assert st == 2 and "128" in msg and "mx_quantize_rowwise_tiled" in msg
    st, msg = _status(L, "mx_quantize_dual_tiled", A16, 1000, 96, None, 0, A16, 4, A16, A16, A16b, A16b, 1152, None)
    assert st == 2 and "128" in msg
    assert _status(L, "mx_quantize_rowwise_tiled", A16, 100, 64 + 1, A16, A16, None)[0] == 2
    assert _status(L, "mx_quantize_rowwise_tiled", A16, 0, 128, None, None, None)[0] == 0    # R == 0: no-op
    assert _status(L, "mx_quantize_rowwise_tiled", A16, 100, 128, A16, None, None)[0] == 1
    for fn in ("mx_grouped_gemm_fwd_tiled", "mx_grouped_gemm_fwd_tiled_fp8feed"):
        st, msg = _status(L, fn, A16, A16, A16b, A16b, A16, 4, 1024, 500, 256, A16, 0, None)   # N % 128
        assert st == 2 and fn in msg, (fn, msg)
        assert _status(L, fn, A16, A16, A16b, A16b, None, 4, 1024, 512, 256, A16, 0, None)[0] == 1


def test_pow2_blockwise_entry_points_validate_like_the_blockwise_ones():
    _, L = _lib()
    ok_args = (A16, A16, A16b, A16b, A16, 4, 1024, 512, 256, A16, 0, None)
    for fn in ("fp8bw_grouped_gemm_fwd_pow2", "fp8bw_grouped_gemm_fwd_pow2_fp8feed", "fp8bw_grouped_gemm_dgrad_pow2",
               "fp8bw_grouped_gemm_dgrad_pow2_fp8feed"):
        a = list(ok_args); a[7] = 500                 # N not a multiple of 128
        st, msg = _status(L, fn, *a)
        assert st == 2 and fn in msg, (fn, msg)
        a = list(ok_args); a[10] = 0x101               # output dtype
        assert _status(L, fn, *a)[0] == 4
        a = list(ok_args); a[3] = BAD                  # B scales not 4-byte aligned
        assert _status(L, fn, *a)[0] == 3
        a = list(ok_args); a[6] = 0                    # M == 0: no-op
        assert _status(L, fn, *a) == (0, "")
    for fn in ("fp8bw_grouped_gemm_wgrad_pow2", "fp8bw_grouped_gemm_wgrad_pow2_fp8feed"):
        # fp8bw_colwise_ld_min(1024, 4) = 1536: 1568 is not a multiple of 128, 1408 is too small
        st, msg = _status(L, fn, A16, A16, A16b, A16b, 1568, A16, 4, 1024, 512, 256, A16, 0, None)
        assert st == 2 and fn in msg and "128" in msg, (fn, msg)
        assert _status(L, fn, A16, A16, A16b, A16b, 1408, A16, 4, 1024, 512, 256, A16, 0, None)[0] == 2
        assert _status(L, fn, A16, A16, A16b, BAD, 1536, A16, 4, 1024, 512, 256, A16, 0, None)[0] == 3


def test_binding_refuses_cpu_tensors():
    m, _ = _lib()
    import torch
    with pytest.raises(ValueError):
        m.mx_quantize_rowwise(torch.zeros((4, 32), dtype=torch.bfloat16))
