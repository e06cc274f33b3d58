/*
 * mxmoe.h -- C ABI of the MXFP8 expert-GEMM library for AMD Instinct MI355X (gfx950).
 *
 * What it computes (sources are the web pages the method is described on):
 *
 *  - MX quantisation: opensourcebeat.com, "Enabling up to 41% faster
 *    pre-training: MXFP8 and DeepEP for DeepSeek-V3 on B200 with TorchTitan",
 *    FAQ "What is MXFP8?": blocks of 32 elements share one exponent.  Element
 *    format E4M3-FN, scale format E8M0 (OCP Microscaling Formats v1.0).
 *    Scale rule (a reading; the page gives none): e = floor(log2 amax) - 8,
 *    e = -127 for an all-zero block, clamped to [-127, 127], stored as e + 127;
 *    elements are E4M3(v * 2^-e), round-to-nearest-even, saturating at +-448,
 *    sign kept (a negative value that rounds to zero is 0x80).
 *  - Dropless grouped GEMM: iitak.ru, "NVIDIA sped up training of
 *    mixture-of-experts models on JAX tenfold": all experts in one call, each
 *    on its real token count, with no capacity padding and no dropped tokens.
 *  - Blockwise FP8: aifind.ru, "DeepSeek-V3: a revolutionary high-performance
 *    language model with low training cost", section "Low-precision training:
 *    FP8 Framework": 1x128 activation tiles and 128x128 weight blocks with their
 *    own scales, partial sums promoted every 128 elements of the contraction.
 *
 * Conventions for every entry point below:
 *  - All tensor pointers are DEVICE pointers of the current HIP device; every
 *    tensor is dense and row-major.  bf16 inputs are passed as raw bit patterns
 *    (`const void*`).  The caller owns and allocates every buffer; the library
 *    never allocates, keeps no state between calls and may be called
 *    concurrently on different streams.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous; group offsets stay on the device and are never read by the
 *    host (no synchronisation), except in mxmoe_check_offsets().
 *  - Arguments are validated on the host before any HIP call; on error nothing
 *    is launched and a status != MXMOE_OK is returned, with a message from
 *    mxmoe_last_error() (thread-local, valid until the next call on the
 *    thread).  No function throws or aborts.
 *  - Offsets: int32 offs[G+1], offs[0] = 0, non-decreasing, offs[G] = M; rows of
 *    the token tensors are sorted by expert.  Invalid device offsets cannot be
 *    detected without a synchronisation: kernels clamp them into [0, M] so no
 *    access leaves the buffers, and the results are then unspecified.
 *  - Pointers must be 16-byte aligned (4-byte for scale arrays).
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXMOE_ABI_VERSION 5

typedef enum {
  MXMOE_OK = 0,
  MXMOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MXMOE_ERR_SHAPE = 2,       /* negative / inconsistent / unsupported sizes */
  MXMOE_ERR_ALIGN = 3,       /* pointer or leading dimension misaligned */
  MXMOE_ERR_DTYPE = 4,       /* unknown output dtype */
  MXMOE_ERR_OFFSETS = 5,     /* offsets rejected by mxmoe_check_offsets */
  MXMOE_ERR_HIP = 6,         /* a HIP call or kernel launch failed */
  MXMOE_ERR_UNSUPPORTED = 7  /* the current device is not gfx950 */
} mxmoe_status;

typedef enum { MXMOE_F32 = 0, MXMOE_BF16 = 1 } mxmoe_dtype;   /* GEMM output dtype */

/* ABI version of the loaded library (MXMOE_ABI_VERSION). */
int mxmoe_abi_version(void);

/* Message describing the last error on the calling thread ("" after success). */
const char* mxmoe_last_error(void);

/* Smallest leading dimension of a column-wise (group-blocked) copy of an
 * [M, C] tensor split into G groups: 32*ceil((M + 31*G)/32).  Pure host
 * arithmetic; returns -1 for M < 0 or G < 1. */
int64_t mx_colwise_ld_min(int64_t M, int32_t G);

/* mxmoe_pitch: the row pitch (bytes of one qT row: ld for E4M3 codes, ld / 2 for
 * E2M1) this library recommends for a column-wise output whose minimum is min_ld
 * bytes: min_ld rounded up to a multiple of 128 (the weight-gradient GEMM then
 * reads the scale rows, ld / 32 bytes, as aligned words straight into LDS), then
 * raised in steps of 1024 while it has the form 2^p + 2^(p-k), k in {7, 8, 9}.
 * Measured on MI355X, the column-wise and dual-layout quantisers write such
 * pitches 15-25% slower: with the DeepSeek-V3-671B expert shard's minimum
 * 65792 = 2^16 + 2^8 the dual launch runs at 4.2 TB/s, at 5.1 TB/s with
 * 65792 + 1024.  A performance hint only: any ld >= the minimum is valid.  Pure
 * host arithmetic; returns -1 for min_ld < 0. */
int64_t mxmoe_pitch(int64_t min_ld);

/* ---------------------------------------------------------------- MX quantise
 * mx_quantize_rowwise: x bf16 [R, C] -> q E4M3 [R, C], s E8M0 [R, C/32].
 * Blocks are 32 consecutive elements of a row (the contraction axis of the
 * consuming GEMM).  R >= 0, C > 0, C % 32 == 0.  Used for X and W (forward)
 * and dY (dgrad).  R == 0 is a no-op. */
mxmoe_status mx_quantize_rowwise(const void* x_bf16, int64_t R, int64_t C,
                                 uint8_t* q, uint8_t* s, void* stream);

/* mx_quantize_colwise: x bf16 [R, C] -> qT E4M3 [C, ld], sT E8M0 [C, ld/32].
 * Blocks are 32 consecutive rows of one column and restart at each group's
 * first row (a reading: the pages show only the forward pass).  Group g's rows
 * go to columns [c_g, c_g + m_g), c_g = 32 * sum_{h<g} ceil(m_h/32); a group's
 * last block may be short (its amax covers real rows only); the <= 31 pad
 * columns after each group, the tail columns and all unused scale bytes are
 * written 0x00.  offs == NULL means one group of R rows (then G is ignored and
 * ld >= 32*ceil(R/32)); otherwise ld >= mx_colwise_ld_min(R, G).  ld % 32 == 0,
 * C % 32 == 0.  Used for dY and X (wgrad, with the routing offsets) and for W
 * viewed as [G*N, K] (dgrad, offs == NULL since N % 32 == 0). */
mxmoe_status mx_quantize_colwise(const void* x_bf16, int64_t R, int64_t C,
                                 const int32_t* offs, int32_t G,
                                 uint8_t* qT, uint8_t* sT, int64_t ld, void* stream);

/* mx_quantize_dual: both layouts of one tensor from a single read of it (the
 * input side of a layer's forward and backward needs X, dY and W both
 * row-wise and column-wise; one pass moves 2 + 2 + 2/32 bytes per element
 * instead of 2 * (2 + 1 + 1/32)).  Results are byte-identical to
 * mx_quantize_rowwise(x') into q [R, C] / s [R, C/32] plus
 * mx_quantize_colwise(x', offs, G, ld) into qT / sT, where x' [R, C] is:
 *   - row_idx == NULL: x itself (R_src ignored);
 *   - otherwise the routed rows x'[r] = x[row_idx[r]] of x [R_src, C] (the
 *     token permute of a dropless MoE layer folded into the quantiser; indices
 *     are read on the device and clamped into [0, R_src)).
 * With offs, every row in [0, offs[G]) is written row-wise; offs[G] == R is
 * required for the whole of q / s to be defined (only the opt-in validator can
 * check device offsets).  Shapes, alignment and errors as the two routines. */
mxmoe_status mx_quantize_dual(const void* x_bf16, int64_t R, int64_t C,
                              const int32_t* row_idx, int64_t R_src,
                              const int32_t* offs, int32_t G,
                              uint8_t* q, uint8_t* s,
                              uint8_t* qT, uint8_t* sT, int64_t ld, void* stream);

/* ---------------------------------------------------------------- MX grouped GEMM
 * Each routine computes, for every expert g in ONE launch, a matrix product
 * over the expert's real rows, from MX operands (value = E4M3 * 2^(E8M0-127)),
 * accumulating in fp32 and writing fp32 or bf16 (round-to-nearest-even).
 * Shapes: N % 128 == 0 and K % 128 == 0.  1 <= G <= 1024.  A tile addresses
 * its operand rows as 32-bit offsets: a row stride (K, N or the leading
 * dimension, in bytes) at which 256 rows span 2 GiB or more is refused with
 * MXMOE_ERR_SHAPE.
 * Operand feed and accuracy:
 *  - these entry points (precise feed): each 32-block is widened exactly to bf16
 *    with its scale folded in and multiplied on the bf16 MFMA, whose sums are
 *    fp32-accurate: |err| <= 1e-5 * sum_k |a_k b_k| per element (as long as no
 *    product underflows fp32);
 *  - the *_fp8feed entry points further below: the block-scaled FP8 MFMA at
 *    twice the rate, with sums truncated per run of products (documented there).
 *
 * fwd:   Y[r, n] = sum_k X[r, k] W[g*N + n, k]          for r in group g
 *        qx/sx = mx_quantize_rowwise(X [M, K]); qw/sw = mx_quantize_rowwise(W [G*N, K]);
 *        y [M, N] (ydt).  M == 0 is a no-op. */
mxmoe_status mx_grouped_gemm_fwd(const uint8_t* qx, const uint8_t* sx,
                                 const uint8_t* qw, const uint8_t* sw,
                                 const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                 void* y, mxmoe_dtype ydt, void* stream);

/* fwd with the gated activation fused into the epilogue (the output side of an expert MLP):
 * W [G*N, K] holds each expert's gate rows [g N, g N + H) and up rows [g N + H, (g+1) N), N = 2H.
 *   y  bf16 [M, N]: the pre-activations Y = X W_g^T (kept for the backward pass);
 *   qh [M, H], sh [M, H/32]: H = silu(gate) * up, silu(z) = z / (1 + e^-z), formed in fp32 from the
 *      GEMM's fp32 sums (hardware exponential and reciprocal: a few ulp relative) and MX-quantised
 *      row-wise (the forward operand of the down GEMM) without H
 *      ever reaching memory in a wider format (a reading: the pages name no activation; SwiGLU is
 *      the gated unit of the DeepSeek-V3 / Llama-4 expert MLPs);
 *   h  f32 [M, H] or NULL: H as formed before quantisation (for checking);
 *   qhT [H, ldh], shT [H, ldh/32], or both NULL: the same fp32 H MX-quantised column-wise, the
 *      weight-gradient operand of the down GEMM, in the layout of mx_quantize_colwise with the
 *      routing offsets (32-row blocks restarting at each expert, pads and the tail 0x00); ldh % 32
 *      == 0 and ldh >= mx_colwise_ld_min(M, G).  Both copies of H leave the epilogue, so H never
 *      reaches memory in a wider format and is not read back to be quantised.
 * Precise feed; N % 256 == 0; qx/sx, qw/sw and offs as for mx_grouped_gemm_fwd.  M == 0 is a no-op
 * (nothing is written). */
mxmoe_status mx_grouped_gemm_fwd_swiglu(const uint8_t* qx, const uint8_t* sx,
                                        const uint8_t* qw, const uint8_t* sw,
                                        const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                        void* y, uint8_t* qh, uint8_t* sh, float* h,
                                        uint8_t* qhT, uint8_t* shT, int64_t ldh, void* stream);

/* dgrad: dX[r, k] = sum_n dY[r, n] W[g*N + n, k]        for r in group g
 *        qdy/sdy = mx_quantize_rowwise(dY [M, N]);
 *        qwT/swT = mx_quantize_colwise(W [G*N, K], offs = NULL) with leading
 *        dimension ldw >= G*N (ldw % 32 == 0); dx [M, K] (dxdt). */
mxmoe_status mx_grouped_gemm_dgrad(const uint8_t* qdy, const uint8_t* sdy,
                                   const uint8_t* qwT, const uint8_t* swT, int64_t ldw,
                                   const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                   void* dx, mxmoe_dtype dxdt, void* stream);

/* wgrad: dW[g, n, k] = sum_{j < m_g} dY_g[j, n] X_g[j, k]   (contraction length m_g
 *        varies per expert; dW_g = 0 for an empty expert, written)
 *        qdyT/sdyT = mx_quantize_colwise(dY [M, N], offs, ld);
 *        qxT/sxT   = mx_quantize_colwise(X  [M, K], offs, ld) with the same ld;
 *        dw [G, N, K] (dwdt).  With ld % 128 == 0 (as mxmoe_pitch returns) the
 *        scale rows are aligned words and both E4M3 feeds load them straight
 *        into LDS; other ld stage them through registers (slower, same result). */
mxmoe_status mx_grouped_gemm_wgrad(const uint8_t* qdyT, const uint8_t* sdyT,
                                   const uint8_t* qxT, const uint8_t* sxT, int64_t ld,
                                   const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                   void* dw, mxmoe_dtype dwdt, void* stream);

/* ---------------------------------------------------------------- full-rate FP8 operand feed
 * The same three products, arguments, layouts, validation and errors as
 * mx_grouped_gemm_fwd / _dgrad / _wgrad, computed on the block-scaled FP8 MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4, E8M0 scales applied by the instruction) at
 * twice the bf16 rate.  Its sums are not fp32-accurate.  Measured on gfx950 (the
 * 16x16x128 and 32x32x64 block-scaled forms and the older FP8 MFMAs alike): the
 * products of each run of 8 consecutive contraction elements held in one lane's
 * 8-byte register group are truncated toward zero to multiples of 2^(E - 13),
 * E = floor(log2) of the run's largest |product|; the runs' sums and the
 * accumulator then add at fp32.  So |err| <= 7 * 2^-13 * sum_runs max|a_k b_k|
 * (+ fp32 rounding) <= 2^-10 * sum_k |a_k b_k|, above the precise feed's bound
 * whenever a run holds products of very different size. */
mxmoe_status mx_grouped_gemm_fwd_fp8feed(const uint8_t* qx, const uint8_t* sx,
                                         const uint8_t* qw, const uint8_t* sw,
                                         const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                         void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status mx_grouped_gemm_dgrad_fp8feed(const uint8_t* qdy, const uint8_t* sdy,
                                           const uint8_t* qwT, const uint8_t* swT, int64_t ldw,
                                           const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                           void* dx, mxmoe_dtype dxdt, void* stream);
mxmoe_status mx_grouped_gemm_wgrad_fp8feed(const uint8_t* qdyT, const uint8_t* sdyT,
                                           const uint8_t* qxT, const uint8_t* sxT, int64_t ld,
                                           const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                           void* dw, mxmoe_dtype dwdt, void* stream);

/* ---------------------------------------------------------------- 128-byte tiled column-wise layout
 * A layout option for the column-wise E4M3 copies (an addition of this library: the pages fix what a
 * column-wise copy holds, not how it is laid out).  The bytes of a copy qT [C, ld] (row c = column c
 * of the source, byte j = group-blocked position j, as mx_quantize_colwise defines them) are stored as
 * ld / 128 tiles of C x 128 bytes:
 *     byte (c, j)  at  (j / 128) * C * 128 + c * 128 + (j % 128),      ld % 128 == 0,
 * so one 128-byte slice of the contraction for all C rows is one contiguous block of memory: the
 * quantiser writes whole tiles, and the GEMMs load a 128-byte stage of a row from one place.  Every
 * scale buffer of this family, column-wise sT [C, ld/32] and row-wise s [R, C/32] alike, is tiled the
 * same way, four bytes (the scales of one 128-element slice) per row and tile:
 *     scale byte (row, b)  at  (b / 4) * rows * 4 + row * 4 + (b % 4),
 * i.e. sT as [ld/128][C][4] and s as [C/128][R][4] (C % 128 == 0), so a quantiser workgroup writes
 * its scale bytes as contiguous runs rather than one piece per row, and a GEMM stage reads the four
 * scale bytes of its 256 rows as one contiguous 1 KiB.  The codes q of a row-wise copy stay row-major.
 * Every buffer keeps its size.
 * Each entry point below takes exactly the arguments, and validates them as, its row-major namesake,
 * with ld (ldh, ldw) % 128 == 0 (MXMOE_ERR_ALIGN for the quantisers, MXMOE_ERR_SHAPE for the GEMMs)
 * and, for a row-wise copy, C % 128 == 0 (MXMOE_ERR_SHAPE) required in addition; results are the same
 * bytes / values permuted as above:
 *   mx_quantize_rowwise_tiled                           s tiled ([C/128][R][4]);
 *   mx_quantize_colwise_tiled                           qT, sT tiled ([ld/128][C][128], [ld/128][C][4]);
 *   mx_quantize_dual_tiled                              qT, sT and s tiled;
 *   mx_grouped_gemm_fwd_tiled[_fp8feed]                 sx, sw tiled ([K/128][M][4], [K/128][G N][4]);
 *   mx_grouped_gemm_fwd_swiglu_tiled                    sx, sw tiled; sh, qhT, shT written tiled
 *                                                       ([H/128][M][4], [ldh/128][H][128],
 *                                                       [ldh/128][H][4]); qhT and shT are required;
 *   mx_grouped_gemm_dgrad_tiled[_fp8feed]               sdy ([N/128][M][4]), qwT, swT ([ldw/128][K][128],
 *                                                       [ldw/128][K][4]) tiled;
 *   mx_grouped_gemm_wgrad_tiled[_fp8feed]               qdyT, sdyT and qxT, sxT tiled
 *                                                       ([ld/128][N][128], [.][N][4]; [ld/128][K][128],
 *                                                       [.][K][4]).
 * The GEMM results are bit-identical to the row-major entry points on the same data (the same
 * products are summed in the same order). */
mxmoe_status mx_quantize_rowwise_tiled(const void* x_bf16, int64_t R, int64_t C,
                                       uint8_t* q, uint8_t* s, void* stream);
mxmoe_status mx_quantize_colwise_tiled(const void* x_bf16, int64_t R, int64_t C,
                                       const int32_t* offs, int32_t G,
                                       uint8_t* qT, uint8_t* sT, int64_t ld, void* stream);
mxmoe_status mx_quantize_dual_tiled(const void* x_bf16, int64_t R, int64_t C,
                                    const int32_t* row_idx, int64_t R_src,
                                    const int32_t* offs, int32_t G,
                                    uint8_t* q, uint8_t* s,
                                    uint8_t* qT, uint8_t* sT, int64_t ld, void* stream);
mxmoe_status mx_grouped_gemm_fwd_tiled(const uint8_t* qx, const uint8_t* sx,
                                       const uint8_t* qw, const uint8_t* sw,
                                       const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                       void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status mx_grouped_gemm_fwd_tiled_fp8feed(const uint8_t* qx, const uint8_t* sx,
                                               const uint8_t* qw, const uint8_t* sw,
                                               const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                               void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status mx_grouped_gemm_fwd_swiglu_tiled(const uint8_t* qx, const uint8_t* sx,
                                              const uint8_t* qw, const uint8_t* sw,
                                              const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                              int64_t K, void* y, uint8_t* qh, uint8_t* sh, float* h,
                                              uint8_t* qhT, uint8_t* shT, int64_t ldh, void* stream);
mxmoe_status mx_grouped_gemm_dgrad_tiled(const uint8_t* qdy, const uint8_t* sdy,
                                         const uint8_t* qwT, const uint8_t* swT, int64_t ldw,
                                         const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                         void* dx, mxmoe_dtype dxdt, void* stream);
mxmoe_status mx_grouped_gemm_dgrad_tiled_fp8feed(const uint8_t* qdy, const uint8_t* sdy,
                                                 const uint8_t* qwT, const uint8_t* swT, int64_t ldw,
                                                 const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                                 int64_t K, void* dx, mxmoe_dtype dxdt, void* stream);
mxmoe_status mx_grouped_gemm_wgrad_tiled(const uint8_t* qdyT, const uint8_t* sdyT,
                                         const uint8_t* qxT, const uint8_t* sxT, int64_t ld,
                                         const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                         void* dw, mxmoe_dtype dwdt, void* stream);
mxmoe_status mx_grouped_gemm_wgrad_tiled_fp8feed(const uint8_t* qdyT, const uint8_t* sdyT,
                                                 const uint8_t* qxT, const uint8_t* sxT, int64_t ld,
                                                 const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                                 int64_t K, void* dw, mxmoe_dtype dwdt, void* stream);

/* ---------------------------------------------------------------- MXFP4
 * The MX scheme with E2M1 elements (OCP MX v1.0 "MXFP4": sign, 2 exponent bits,
 * 1 mantissa bit, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): the pages announce a
 * 4-bit format as the next step after MXFP8; on gfx950 the block-scaled MFMA runs
 * it at twice the FP8 rate.  Scale e = floor(log2 amax) - 2 clamped to
 * [-127, 127] (byte e + 127), codes E2M1(v * 2^-e) to nearest even, saturating
 * at 6.  Codes are packed two per byte along the contraction axis, element 2i in
 * the low nibble of byte i.  Layouts, offsets and errors as the E4M3 routines
 * with byte counts halved: row-wise q [R, C/2], column-wise qT [C, ld/2]. */
mxmoe_status mxfp4_quantize_rowwise(const void* x_bf16, int64_t R, int64_t C,
                                    uint8_t* q, uint8_t* s, void* stream);
mxmoe_status mxfp4_quantize_colwise(const void* x_bf16, int64_t R, int64_t C,
                                    const int32_t* offs, int32_t G,
                                    uint8_t* qT, uint8_t* sT, int64_t ld, void* stream);

/* MXFP4 grouped GEMMs: the same products as mx_grouped_gemm_* over packed E2M1
 * operands (from the mxfp4 quantisers; ldw and ld count elements, as for E4M3).
 * They always use the block-scaled MFMA (E2M1 format): every E2M1 product is a
 * multiple of 1/4 below 36 times its pair of scales, which the instruction sums
 * exactly, so |err| <= 1e-5 * sum_k |a_k b_k| as for the precise E4M3 feed.
 * N % 256 == 0 and K % 256 == 0. */
mxmoe_status mxfp4_grouped_gemm_fwd(const uint8_t* qx, const uint8_t* sx,
                                    const uint8_t* qw, const uint8_t* sw,
                                    const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                    void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status mxfp4_grouped_gemm_dgrad(const uint8_t* qdy, const uint8_t* sdy,
                                      const uint8_t* qwT, const uint8_t* swT, int64_t ldw,
                                      const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                      void* dx, mxmoe_dtype dxdt, void* stream);
mxmoe_status mxfp4_grouped_gemm_wgrad(const uint8_t* qdyT, const uint8_t* sdyT,
                                      const uint8_t* qxT, const uint8_t* sxT, int64_t ld,
                                      const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                      void* dw, mxmoe_dtype dwdt, void* stream);

/* ---------------------------------------------------------------- blockwise FP8
 * The GEMMs have the same accuracy as the MX GEMMs (precise feed), and
 * *_fp8feed forms (the full-rate FP8 feed described above).  Scale rule (a reading): s = fl32(amax / 448) by IEEE fp32 division, s = 1 for
 * an all-zero tile; q = E4M3(fl32(v / s)), nearest-even, saturating.
 *
 * fp8bw_quantize_act_1x128: x bf16 [R, C] -> q [R, C], s f32 [R, C/128]
 * (one scale per row and 128 consecutive columns).  C % 128 == 0. */
mxmoe_status fp8bw_quantize_act_1x128(const void* x_bf16, int64_t R, int64_t C,
                                      uint8_t* q, float* s, void* stream);

/* fp8bw_quantize_weight_128x128: w bf16 [R, C] (R = G*N) -> q [R, C],
 * s f32 [R/128, C/128] (amax over each 128x128 block).  R % 128 == 0, C % 128 == 0.
 * qT, if not NULL, also receives the codes transposed, qT [C, R] (qT[c, r] = q[r, c]): the weight
 * operand of fp8bw_grouped_gemm_dgrad, which contracts over the rows of W (same block scales). */
mxmoe_status fp8bw_quantize_weight_128x128(const void* w_bf16, int64_t R, int64_t C,
                                           uint8_t* q, float* s, uint8_t* qT, void* stream);

/* fp8bw_grouped_gemm_fwd: Y[r, n] = sum_kb sx[r, kb] sw[(gN+n)/128, kb] *
 *                                   sum_{k in kb} qx[r, k] qw[gN+n, k]
 * (FP8 products summed over each 128-slice, then promoted in fp32).
 * qx/sx from fp8bw_quantize_act_1x128(X [M, K]); qw/sw from
 * fp8bw_quantize_weight_128x128(W [G*N, K]).  N % 128 == 0, K % 128 == 0. */
mxmoe_status fp8bw_grouped_gemm_fwd(const uint8_t* qx, const float* sx,
                                    const uint8_t* qw, const float* sw,
                                    const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                    void* y, mxmoe_dtype ydt, void* stream);

/* fp8bw_grouped_gemm_dgrad: dX[r, k] = sum_nb sdy[r, nb] sw[gN/128 + nb, k/128] *
 *                                      sum_{n in nb} qdy[r, n] qwT[k, gN+n]
 * qdy/sdy from fp8bw_quantize_act_1x128(dY [M, N]) (1x128 along N); qwT [K, G*N] is the transposed
 * weight copy from fp8bw_quantize_weight_128x128 and sw its (forward-layout) block scales: the
 * 128x128 weight blocks of the forward pass, read transposed.  dx [M, K]. */
mxmoe_status fp8bw_grouped_gemm_dgrad(const uint8_t* qdy, const float* sdy,
                                      const uint8_t* qwT, const float* sw,
                                      const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                      void* dx, mxmoe_dtype dxdt, void* stream);

/* fp8bw_grouped_gemm_fwd_pow2 / fp8bw_grouped_gemm_dgrad_pow2: the same products (arguments, layouts
 * and errors as fp8bw_grouped_gemm_fwd / _dgrad) for scales that are powers of two, as the _pow2
 * quantisers write them.  Such a scale is exactly representable as an E8M0 byte, so each 128-slice
 * is multiplied exactly with its scales folded into the operands and summed in the fp32 accumulator
 * across the whole contraction (the MX kernel): the promoted sum of the recipe and this sum differ
 * only in fp32 rounding order, within the same |err| <= 1e-5 * sum |a b| bound.  A scale that is not
 * a power of two is read as the power of two of its exponent (a wrong result, not an error: the
 * scales are device data).  The _fp8feed forms use the block-scaled FP8 MFMA. */
mxmoe_status fp8bw_grouped_gemm_fwd_pow2(const uint8_t* qx, const float* sx,
                                         const uint8_t* qw, const float* sw,
                                         const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                         void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status fp8bw_grouped_gemm_dgrad_pow2(const uint8_t* qdy, const float* sdy,
                                           const uint8_t* qwT, const float* sw,
                                           const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                           void* dx, mxmoe_dtype dxdt, void* stream);
mxmoe_status fp8bw_grouped_gemm_fwd_pow2_fp8feed(const uint8_t* qx, const float* sx,
                                                 const uint8_t* qw, const float* sw,
                                                 const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                                 void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status fp8bw_grouped_gemm_dgrad_pow2_fp8feed(const uint8_t* qdy, const float* sdy,
                                                   const uint8_t* qwT, const float* sw,
                                                   const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                                   void* dx, mxmoe_dtype dxdt, void* stream);
/* fp8bw_grouped_gemm_wgrad_pow2[_fp8feed]: fp8bw_grouped_gemm_wgrad (arguments, layouts and errors as
 * declared below) for power-of-two scales, on the same footing as the two above. */
mxmoe_status fp8bw_grouped_gemm_wgrad_pow2(const uint8_t* qdyT, const float* sdyT,
                                           const uint8_t* qxT, const float* sxT, int64_t ld,
                                           const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                           void* dw, mxmoe_dtype dwdt, void* stream);
mxmoe_status fp8bw_grouped_gemm_wgrad_pow2_fp8feed(const uint8_t* qdyT, const float* sdyT,
                                                   const uint8_t* qxT, const float* sxT, int64_t ld,
                                                   const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                                   int64_t K, void* dw, mxmoe_dtype dwdt, void* stream);

/* Full-rate FP8 operand feed of the blockwise GEMMs (arguments as above; accuracy as the MX
 * *_fp8feed routines, each 128-slice partial truncated per run of products before its promotion). */
mxmoe_status fp8bw_grouped_gemm_fwd_fp8feed(const uint8_t* qx, const float* sx,
                                            const uint8_t* qw, const float* sw,
                                            const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                            void* y, mxmoe_dtype ydt, void* stream);
mxmoe_status fp8bw_grouped_gemm_dgrad_fp8feed(const uint8_t* qdy, const float* sdy,
                                              const uint8_t* qwT, const float* sw,
                                              const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                              void* dx, mxmoe_dtype dxdt, void* stream);

/* fp8bw_colwise_ld_min: smallest leading dimension of the column-wise blockwise
 * layout for M rows in G groups, 128 * ceil((M + 127 G) / 128) (-1 for M < 0 or
 * G < 1).  Host-only arithmetic. */
int64_t fp8bw_colwise_ld_min(int64_t M, int32_t G);

/* fp8bw_quantize_colwise_128: x bf16 [R, C] -> qT E4M3 [C, ld], sT f32 [C, ld/128].
 * The weight-gradient operands of the blockwise recipe (a reading: the page shows
 * the forward pass only; the backward pass quantises along its own contraction
 * axis, the tokens of one expert): blocks of 128 consecutive rows of one column,
 * restarting at each group's first row, scale s = fl32(amax / 448) (1 for an
 * all-zero block), codes E4M3(fl32(v / s)).  Group g occupies columns
 * [c_g, c_g + m_g), c_g = 128 * sum_{h<g} ceil(m_h/128); a group's last block may
 * be short (amax over real rows); pad and tail bytes are 0x00 and scale slots of
 * no block are 0.  offs == NULL means one group of R rows (ld >= 128*ceil(R/128));
 * otherwise ld >= fp8bw_colwise_ld_min(R, G).  ld % 128 == 0, C % 128 == 0. */
mxmoe_status fp8bw_quantize_colwise_128(const void* x_bf16, int64_t R, int64_t C,
                                        const int32_t* offs, int32_t G,
                                        uint8_t* qT, float* sT, int64_t ld, void* stream);

/* Power-of-two scale mode of the three blockwise quantisers (aifind.ru DeepSeek-V3 article, section
 * "Low-precision training: FP8 Framework" fixes the 1x128 / 128x128 tiles and fp32 scales only; this
 * optional mode is a reading): each tile's scale is the smallest power of two s with 448 s >= amax,
 * at least 2^-126, and 1 for an all-zero tile; codes E4M3(v / s) (an exact division), so no element
 * saturates.  Same arguments, layouts, validation and errors as the functions above; the outputs
 * feed the same blockwise GEMMs. */
mxmoe_status fp8bw_quantize_act_1x128_pow2(const void* x_bf16, int64_t R, int64_t C,
                                           uint8_t* q, float* s, void* stream);
mxmoe_status fp8bw_quantize_weight_128x128_pow2(const void* w_bf16, int64_t R, int64_t C,
                                                uint8_t* q, float* s, uint8_t* qT, void* stream);
mxmoe_status fp8bw_quantize_colwise_128_pow2(const void* x_bf16, int64_t R, int64_t C,
                                             const int32_t* offs, int32_t G,
                                             uint8_t* qT, float* sT, int64_t ld, void* stream);

/* fp8bw_grouped_gemm_wgrad: dW[g, n, k] = sum_b sdyT[n, c_g/128 + b] sxT[k, c_g/128 + b] *
 *                                         sum_{j in block b} qdyT[n, j] qxT[k, j]
 * over expert g's 128-token blocks b (each block's FP8 partial promoted with its two
 * fp32 scales).  qdyT/sdyT = fp8bw_quantize_colwise_128(dY [M, N], offs, ld),
 * qxT/sxT = fp8bw_quantize_colwise_128(X [M, K], offs, ld) with the same ld;
 * dw [G, N, K] (dwdt); dW_g = 0 for an empty expert, written (also for M == 0). */
mxmoe_status fp8bw_grouped_gemm_wgrad(const uint8_t* qdyT, const float* sdyT,
                                      const uint8_t* qxT, const float* sxT, int64_t ld,
                                      const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                      void* dw, mxmoe_dtype dwdt, void* stream);
mxmoe_status fp8bw_grouped_gemm_wgrad_fp8feed(const uint8_t* qdyT, const float* sdyT,
                                              const uint8_t* qxT, const float* sxT, int64_t ld,
                                              const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                              void* dw, mxmoe_dtype dwdt, void* stream);

/* Opt-in offsets validator: copies offs to the host (synchronising `stream`)
 * and checks offs[0] == 0, non-decreasing, offs[G] == M.  Returns
 * MXMOE_ERR_OFFSETS with a message naming the first bad index. */
mxmoe_status mxmoe_check_offsets(const int32_t* offs, int32_t G, int64_t M, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
