"""CPU oracle for the MXFP8 expert-GEMM hot path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy reference of what the GPU library
computes.  Only the test-suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path (the HIP
library and its Python binding) never imports, links or calls anything here,
and this package imports nothing from the product.

Sources (page title, section), restated rather than quoted:

* opensourcebeat.com, "Enabling up to 41 % faster pre-training: MXFP8 and
  DeepEP for DeepSeek-V3 on B200 with TorchTitan": FAQ "What is MXFP8?" -- a
  block of 32 elements shares one exponent; section "Two-sided attack" --
  MXFP8 is applied to the grouped GEMMs of MoE expert layers.
* iitak.ru, "NVIDIA sped up training of mixture-of-experts models on JAX
  tenfold": dropless routing; the grouped GEMM computes every expert in one
  call on its real token count, with no padding to the maximum.
* aifind.ru, "DeepSeek-V3: a revolutionary high-performance language model
  with low training cost", section "Low-precision training: FP8 Framework":
  activations in 1x128 tiles and weights in 128x128 blocks, each with its own
  scale; partial sums promoted to full precision every 128 elements.

Where the pages are silent (scale rule, rounding, saturation, E4M3 variant,
block direction in backward, group boundaries) the readings are stated in the
docstring of the function that applies them.  Element and scale encodings
follow the OCP Microscaling Formats (MX) v1.0 specification (E4M3 "FN":
bias 7, max 448, no infinities; E8M0: bias 127, 0xFF = NaN).

Parity pins: every exported function is checked against closed forms, a
library routine (torch's CPU float8 cast and float32 division), brute force,
dense products of the dequantised operands or invariants in
``tests/test_oracle_*.py``; the scale rule ``mx_block_exponent`` is pinned
through the quantisers' exhaustive bf16 sweeps.
"""
from .codecs import (E2M1_MAX, e2m1_decode, e2m1_encode, e2m1_encode_bruteforce, fp4_pack, fp4_unpack,
                     E4M3_MAX, bf16_bits_to_f64, e4m3_decode, e4m3_encode,
                     e4m3_encode_bruteforce, e8m0_decode)
from .mx import (mx_block_exponent, mx_colwise_ld_min, mx_dequantize,
                 mx_quantize_colwise, mx_quantize_rowwise, mx_group_columns,
                 mx_gather_rows, mx_quantize_dual, mxfp4_quantize_rowwise,
                 mxfp4_quantize_colwise, mxfp4_dequantize, mx_quantize_rowwise_values,
                 mx_quantize_colwise_values, mx_colwise_tiled, mx_scales_tiled, swiglu)
from .blockwise import (bw_quantize_act_1x128, bw_quantize_weight_128x128,
                        bw_dequantize_act, bw_dequantize_weight, bw_colwise_ld_min,
                        bw_group_columns, bw_quantize_colwise_128, pow2_scale)
from .gemm import (mx_gemm_fwd, mx_gemm_dgrad, mx_gemm_wgrad, bw_gemm_fwd,
                   bw_gemm_dgrad, bw_gemm_wgrad, mxfp4_gemm_fwd, mxfp4_gemm_dgrad, mxfp4_gemm_wgrad, gemm_tolerance, check_gemm)

__all__ = [
    "E4M3_MAX", "bf16_bits_to_f64", "e4m3_decode", "e4m3_encode",
    "e4m3_encode_bruteforce", "e8m0_decode",
    "mx_block_exponent", "mx_colwise_ld_min", "mx_dequantize",
    "mx_quantize_colwise", "mx_quantize_rowwise", "mx_group_columns",
    "bw_quantize_act_1x128", "bw_quantize_weight_128x128", "pow2_scale",
    "bw_dequantize_act", "bw_dequantize_weight",
    "mx_gemm_fwd", "mx_gemm_dgrad", "mx_gemm_wgrad", "bw_gemm_fwd",
    "bw_gemm_dgrad", "gemm_tolerance", "check_gemm",
]
