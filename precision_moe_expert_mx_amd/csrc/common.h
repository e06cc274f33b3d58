// Shared device helpers and internal launch declarations of the MXFP8 expert-GEMM library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxmoe.h"

namespace mxmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// GEMM operand feeds: bf16-widened operands on the bf16 MFMA (fp32-accurate sums), or the
// full-rate block-scaled FP8 MFMA (sums truncated per 8-element run, see gemm_mx.hip).
enum GemmFeed { kFeedPrecise = 0, kFeedFast = 1 };

// ---- memory and lane helpers ---------------------------------------------------------------------
// Non-temporal 16-byte loads and 8 / 4-byte stores for streaming kernels (every byte touched once).
typedef uint32_t v4u_ __attribute__((ext_vector_type(4)));
typedef uint32_t v2u_ __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load16_nt(const uint4* p) {
  const v4u_ v = __builtin_nontemporal_load((const v4u_*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store8_nt(uint2* p, uint2 v) { __builtin_nontemporal_store(v2u_{v.x, v.y}, (v2u_*)p); }
__device__ __forceinline__ void store4_nt(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of the quad ends with the quad's maximum
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
  return m;
}

// Maximum over each group of 8 lanes: quad permutes, then the half-row mirror (lane i of an 8-lane
// group with lane 7 - i, in the other quad).  bound_ctrl with an old value of 0 (the identity of an
// unsigned max) lets each permute fold into the max as one DPP instruction.
__device__ __forceinline__ uint32_t oct_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, true));
  return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, true));
}

// Maximum over each row of 16 lanes: the 8-lane maximum, then the row mirror (lane i with 15 - i).
__device__ __forceinline__ uint32_t hex_max(uint32_t m) {
  m = oct_max(m);
  return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, true));
}

// ---- MX scale helpers (E8M0 shared exponent of a 32-block) -------------------------------------
// The magnitude bits of a finite bf16 value order like the value itself, so amax is an integer max
// over (bits & 0x7FFF).  floor(log2 v) of that magnitude: exponent field - 127 for normals, and for
// subnormals (m * 2^-133) the index of m's leading bit - 133.
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
  uint32_t e = mag >> 7;
  if (e != 0) return (int)e - 127;
  // subnormal (mag != 0 assumed by caller): 31 - clz(m) is the leading-bit index of m
  return (31 - __builtin_clz(mag)) - 133;
}

// Shared exponent e = clamp(floor(log2 amax) - 8, -127, 127), -127 for amax = 0, of a block with
// magnitude bits `amax_bits`.  Branch-free: a normal amax with exponent field E gives E - 135 (at most
// 254 - 135 = 119, so the upper clamp never applies), and a zero or subnormal amax (field 0,
// floor(log2) <= -127) gives at most -135 before clamping, so both reduce to max(E - 135, -127).
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  return max((int)(amax_bits >> 7) - 135, -127);
}

// The same rule for E2M1 elements (largest exponent 2): max(E - 129, -127).
__device__ __forceinline__ int mxfp4_exponent(uint32_t amax_bits) {
  return max((int)(amax_bits >> 7) - 129, -127);
}

// Eight bf16 (four dwords, element order) -> eight E2M1 codes packed two per byte, element 2i in the
// low nibble of byte i.  The conversion divides by the power of two whose exponent field is that of
// `scale`, rounds to nearest even and saturates at 6 (checked on gfx950 against every finite bf16
// at several scales), so no clamp is needed.
__device__ __forceinline__ uint32_t cvt8_e2m1(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, float scale) {
  typedef __bf16 v2bf_ __attribute__((ext_vector_type(2)));
  uint32_t o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(v2bf_, w0), scale, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_, w1), scale, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_, w2), scale, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_, w3), scale, 3);
}

// bf16 bit pattern of 448 * 2^e (the largest magnitude that does not saturate), e in [-127, 119].
__device__ __forceinline__ uint32_t mx_clamp_bits(int e) { return ((uint32_t)(e + 135) << 7) | 0x60u; }

// Convert two bf16 (one dword, low half first) to two E4M3 bytes placed in the low or high
// half-word of `old`.  The magnitude is first clamped to 448 * 2^e so values that would round
// above 448 saturate (the hardware conversion returns NaN on overflow); the conversion divides by
// the power of two whose exponent field is `scale_bits` (only the exponent is used) and rounds to
// nearest even, keeping the sign.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_e4m3(uint32_t old, uint32_t w, uint32_t clamp_pk, float scale) {
  typedef unsigned short v2us __attribute__((ext_vector_type(2)));
  v2us mag = __builtin_bit_cast(v2us, w & 0x7FFF7FFFu);
  v2us lim = __builtin_bit_cast(v2us, clamp_pk);
  uint32_t c = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(mag, lim)) | (w & 0x80008000u);
  v2s o = __builtin_bit_cast(v2s, old);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(v2bf, c), scale, HI);
  return __builtin_bit_cast(uint32_t, o);
}

// Four fp32 values -> four E4M3 bytes with the power-of-two scale `scale`; magnitudes are first
// clamped to lim = 448 * scale so that values rounding above 448 saturate.
__device__ __forceinline__ uint32_t cvt4_f32_e4m3_scaled(float a, float b, float c, float d, float lim, float scale) {
  const float ca = copysignf(fminf(fabsf(a), lim), a), cb = copysignf(fminf(fabsf(b), lim), b);
  const float cc = copysignf(fminf(fabsf(c), lim), c), cd = copysignf(fminf(fabsf(d), lim), d);
  v2s o = v2s{0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, ca, cb, scale, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, cc, cd, scale, true);
  return __builtin_bit_cast(uint32_t, o);
}

// Four bf16 (two dwords) -> four E4M3 bytes.
__device__ __forceinline__ uint32_t cvt4_e4m3(uint32_t w0, uint32_t w1, uint32_t clamp_pk, float scale) {
  uint32_t r = cvt2_e4m3<false>(0u, w0, clamp_pk, scale);
  return cvt2_e4m3<true>(r, w1, clamp_pk, scale);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Device-side clamp of an offset read from memory into [0, M].
__device__ __forceinline__ int64_t clamp_off(int64_t v, int64_t M) { return v < 0 ? 0 : (v > M ? M : v); }

// Column-wise layouts place group g's blocks of BLK rows from block-column starts[g] =
// sum_{h<g} ceil(m_h / BLK).  Wave 0 of the workgroup scans the clamped offsets 64 groups per step and
// writes starts[0..G] and rows0[g] = offs[g] (offs NULL: one group of R rows).  The caller
// synchronises before reading them.
template <int BLK>
__device__ __forceinline__ void group_block_starts(const int32_t* offs, int G, int64_t R, int32_t* starts,
                                                   int32_t* rows0) {
  if (threadIdx.x < 64) {
    int lane = threadIdx.x;
    int32_t carry = 0;
    for (int g0 = 0; g0 <= G; g0 += 64) {
      int g = g0 + lane;
      int32_t nb = 0;
      int64_t o0 = 0;
      if (g <= G) {
        o0 = offs ? clamp_off(offs[g], R) : (g == 0 ? 0 : R);
        rows0[g] = (int32_t)o0;
      }
      if (g < G) {
        int64_t o1 = offs ? clamp_off(offs[g + 1], R) : R;
        int64_t m = o1 > o0 ? o1 - o0 : 0;
        nb = (int32_t)((m + BLK - 1) / BLK);
      }
      // inclusive scan of nb across the wave
      int32_t incl = nb;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int32_t t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
      }
      if (g <= G) starts[g] = carry + incl - nb;    // exclusive
      carry += __shfl(incl, 63, 64);
    }
  }
}

// Block-column bc of a column-wise layout (see group_block_starts): first row r0 and row count n
// (<= BLK) of the block it holds, n = 0 for pad / tail block-columns.
template <int BLK>
__device__ __forceinline__ void block_rows(int bc, int nbc, int G, const int32_t* starts, const int32_t* rows0,
                                           int32_t& r0, int32_t& n) {
  r0 = 0;
  n = 0;
  if (bc < nbc && bc < starts[G]) {
    // last group g with starts[g] <= bc (empty groups share their start with the next group)
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (starts[mid] <= bc) lo = mid; else hi = mid - 1;
    }
    const int64_t g0 = rows0[lo], g1 = rows0[lo + 1];
    r0 = (int32_t)(g0 + (int64_t)BLK * (bc - starts[lo]));
    const int64_t left = g1 - r0;
    n = (int32_t)(left < BLK ? left : BLK);
  }
}

// ---- internal launchers (defined in the .hip files; arguments already validated) ---------------
hipError_t launch_mx_rowwise(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, bool tiled,
                             hipStream_t st);
// tiled: qT and sT in the 128-byte tiled layout, [ld / 128][C][128] and [ld / 128][C][4] (ld % 128 == 0);
// for the row-wise copies (launch_mx_rowwise, launch_mx_dual) s as [C / 128][R][4] (C % 128 == 0)
hipError_t launch_mx_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                             uint8_t* qT, uint8_t* sT, int64_t ld, bool tiled, hipStream_t st);
hipError_t launch_mxfp4_rowwise(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, hipStream_t st);
hipError_t launch_mxfp4_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                                uint8_t* qT, uint8_t* sT, int64_t ld, hipStream_t st);
hipError_t launch_mx_dual(const uint16_t* x, int64_t R, int64_t C, const int32_t* row_idx, int64_t Rsrc,
                          const int32_t* offs, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t ld,
                          bool tiled, hipStream_t st);
hipError_t launch_bw_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G, uint8_t* qT,
                             float* sT, int64_t ld, bool pow2, hipStream_t st);
hipError_t launch_bw_act(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, bool pow2, hipStream_t st);
hipError_t launch_bw_weight(const uint16_t* w, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT, bool pow2,
                            hipStream_t st);

enum GemmMode { kFwd = 0, kDgrad = 1, kWgrad = 2 };

struct GemmArgs {
  const uint8_t* a;   // A operand rows (E4M3), contraction contiguous
  const void* sa;     // A scales: uint8 E8M0 per 32 (MX) or float per 128 (blockwise)
  const uint8_t* b;   // B operand rows
  const void* sb;     // B scales
  const int32_t* offs;
  void* out;
  int64_t lda, ldsa;  // A row stride in bytes / scale row stride in scale elements
  int64_t ldb, ldsb;
  // MX: bytes between consecutive 128-byte contraction chunks of an operand row: 128 in the row-major
  // layouts, rows * 128 in the 128-byte tiled column-wise layout (whose row stride is then 128)
  int64_t a_kstride, b_kstride;
  // MX: bytes between consecutive 4-byte groups of a row's scale bytes (the scales of one 128-element
  // chunk): 4 in the row-major layouts, rows * 4 in the tiled column-wise layout (whose scale row
  // stride ldsa / ldsb is then 4)
  int64_t sa_gstride, sb_gstride;
  // wgrad: leading dimension of the column-wise copies in elements (the expert clip)
  int64_t ld_cols;
  int64_t M, N, K;    // problem sizes as in the ABI
  int32_t G;
  int32_t out_bf16;
  int32_t feed;       // GemmFeed
  int32_t scale_dword;  // MX: every row's scale bytes of a stage form aligned dwords
  int32_t fp4;          // MX operands are E2M1 (two per byte; leading dimensions in bytes)
  int32_t bw_pow2;      // MX kernel on blockwise operands whose fp32 scales are powers of two (fwd, dgrad)
  // forward with the gated activation in the epilogue: out = Y bf16 [M, 2H] (gate | up), plus
  // H = silu(gate) * up MX-quantised row-wise into act_q [M, H] / act_s [M, H/32], and H in fp32 into
  // act_dbg [M, H] when not NULL
  uint8_t* act_q;
  uint8_t* act_s;
  float* act_dbg;
  // and, when act_qT is not NULL, H MX-quantised column-wise (32-row blocks restarting at each expert,
  // the layout of mx_quantize_colwise) into act_qT [H, act_ld] / act_sT [H, act_ld / 32]
  uint8_t* act_qT;
  uint8_t* act_sT;
  int64_t act_ld;
  int32_t act_tiled;    // the tiled layouts: act_qT [act_ld / 128][H][128], act_sT [act_ld / 128][H][4],
                        // act_s [H / 128][M][4]
};

hipError_t launch_mx_gemm(int mode, const GemmArgs& a, hipStream_t st);
hipError_t launch_bw_gemm(int mode, const GemmArgs& a, hipStream_t st);

}  // namespace mxmoe
