// Blockwise ("fine-grained") FP8 quantisers for gfx950: E4M3 elements with one fp32 scale per
// 1x128 activation tile or per 128x128 weight block (aifind.ru DeepSeek-V3 article, section
// "Low-precision training: FP8 Framework").  Scale s = fl32(amax / 448) by IEEE division (1 for an
// all-zero tile); elements E4M3(fl32(v / s)), nearest even.  |v / s| <= 448 (1 + 2^-23)^2 < 464,
// so the hardware conversion (which rounds to nearest even) never overflows and no clamp is needed.
//
// Power-of-two mode (POW2): the scale is instead the smallest power of two s with 448 s >= amax, at
// least 2^-126 (1 for an all-zero tile).  From the bf16 magnitude bits of amax (exponent field E,
// mantissa m): amax / 448 = ((1 + m/128) / 1.75) 2^(E - 135), so e = E - 135, plus 1 when m > 96
// (significand above 1.75); subnormal amax falls below the clamp.  Dividing by s is exact, so it is a
// multiplication by 2^-e.
//
// fl32(v / s) without a division per element: with y = fl32(1 / s), formed once per tile,
//   q0 = fl32(v y),  r = v - s q0 (exact, one FMA),  q = fl32(q0 + r y) (one FMA)
// is the correctly rounded quotient (Markstein's division correction: y within half an ulp of 1/s,
// q0 within an ulp of v/s) as long as the remainder does not underflow.  Checked on the host for every
// bf16 amax >= 2^-59 and every bf16 v with |v| <= amax, both signs, with IEEE and with flushed
// denormals: the E4M3 codes equal those of the IEEE quotient.  v = -0 yields +0 through the FMAs, so
// the sign of v is put back.  Tiles with a smaller amax divide per element.
#include "common.h"

namespace mxmoe {

__device__ __forceinline__ uint32_t cvt4_f32_e4m3(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// A tile's scale s and what its elements are divided with: y = 1 / s (exact in the power-of-two
// mode, fl32(1 / s) otherwise) and whether the tile's amax admits the FMA correction.
struct BwScale {
  float s, y;
  bool fma;
};
constexpr uint32_t kBwFmaMinAmax = 68u << 7;   // bf16 bits of 2^-59

template <bool POW2>
__device__ __forceinline__ BwScale bw_scale(uint32_t m) {
  BwScale r;
  if (POW2) {
    const int e = max((int)(m >> 7) - 135 + ((m & 0x7Fu) > 96u ? 1 : 0), -126);
    r.s = m == 0 ? 1.0f : __uint_as_float((uint32_t)(e + 127) << 23);
    r.y = m == 0 ? 1.0f : __uint_as_float((uint32_t)(127 - e) << 23);
    r.fma = true;
  } else {
    r.s = m == 0 ? 1.0f : __fdiv_rn(__uint_as_float(m << 16), 448.0f);
    r.fma = m >= kBwFmaMinAmax;
    r.y = r.fma ? __fdiv_rn(1.0f, r.s) : 0.0f;
  }
  return r;
}

// fl32(v / s) for an element v of the tile (see the header).
template <bool POW2>
__device__ __forceinline__ float bw_quot(float v, const BwScale& sc) {
  if (POW2) return v * sc.y;
  const float q0 = v * sc.y;
  const float r = __builtin_fmaf(-sc.s, q0, v);
  return __builtin_copysignf(__builtin_fmaf(r, sc.y, q0), v);
}

// Quantise 8 bf16 (one uint4) of one tile -> 8 bytes.
template <bool POW2>
__device__ __forceinline__ uint2 bw_convert8(const uint4& v, const BwScale& sc) {
  uint2 o;
  if (POW2 || sc.fma) {
    o.x = cvt4_f32_e4m3(bw_quot<POW2>(bf16_lo(v.x), sc), bw_quot<POW2>(bf16_hi(v.x), sc),
                        bw_quot<POW2>(bf16_lo(v.y), sc), bw_quot<POW2>(bf16_hi(v.y), sc));
    o.y = cvt4_f32_e4m3(bw_quot<POW2>(bf16_lo(v.z), sc), bw_quot<POW2>(bf16_hi(v.z), sc),
                        bw_quot<POW2>(bf16_lo(v.w), sc), bw_quot<POW2>(bf16_hi(v.w), sc));
  } else {
    const float s = sc.s;
    o.x = cvt4_f32_e4m3(__fdiv_rn(bf16_lo(v.x), s), __fdiv_rn(bf16_hi(v.x), s),
                        __fdiv_rn(bf16_lo(v.y), s), __fdiv_rn(bf16_hi(v.y), s));
    o.y = cvt4_f32_e4m3(__fdiv_rn(bf16_lo(v.z), s), __fdiv_rn(bf16_hi(v.z), s),
                        __fdiv_rn(bf16_lo(v.w), s), __fdiv_rn(bf16_hi(v.w), s));
  }
  return o;
}

// Four elements of one column (bf16 in the low or high half of each dword) of one tile -> 4 codes.
template <bool POW2, bool HI>
__device__ __forceinline__ uint32_t bw_convert4_col(const uint32_t* w, const BwScale& sc) {
  float f[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) f[k] = HI ? bf16_hi(w[k]) : bf16_lo(w[k]);
  if (POW2 || sc.fma) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = bw_quot<POW2>(f[k], sc);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __fdiv_rn(f[k], sc.s);
  }
  return cvt4_f32_e4m3(f[0], f[1], f[2], f[3]);
}

__device__ __forceinline__ uint32_t magmax8(const uint4& v) {
  uint32_t a = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  uint32_t b = max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
  return max(a, b);
}

// 1x128 activation tiles: 16 lanes per tile (16 bytes each, one DPP row), amax reduced by DPP within
// the row.  A workgroup of 512 lanes covers 2 x 512 consecutive 16-byte chunks with non-temporal loads
// and stores (every byte is touched once), the launch shape of the MX row-wise quantiser.
constexpr int kBwActThreads = 512;
constexpr int kBwActUnroll = 2;

template <bool POW2>
__global__ __launch_bounds__(kBwActThreads) void bw_act_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                               uint2* __restrict__ q, float* __restrict__ s) {
  const int64_t base = (int64_t)blockIdx.x * (kBwActThreads * kBwActUnroll) + threadIdx.x;
  uint4 v[kBwActUnroll];
#pragma unroll
  for (int j = 0; j < kBwActUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kBwActThreads;
    v[j] = i < nchunks ? load16_nt(x + i) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kBwActUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kBwActThreads;
    // nchunks is a multiple of 16 and rows are 16-aligned, so a tile is wholly in or out of range
    const BwScale sc = bw_scale<POW2>(hex_max(magmax8(v[j])));
    const uint2 o = bw_convert8<POW2>(v[j], sc);
    if (i < nchunks) {
      store8_nt((uint2*)q + i, o);
      if ((threadIdx.x & 15) == 0) s[i >> 4] = sc.s;
    }
  }
}

// 128x128 weight blocks: one workgroup of 256 lanes per block; lane t owns rows (t/16) + 16 i,
// 16-byte column chunk t%16, i = 0..7 (64 values in registers), amax reduced through LDS.  When qT is
// given, the block's codes also go through an LDS tile and out transposed (qT [C, R], 128-byte rows),
// the operand layout of the dgrad GEMM, which contracts over the rows.
constexpr int kBwTPitch = 128 + 16;     // LDS bytes per transposed row (padded against bank conflicts)

template <bool POW2>
__global__ __launch_bounds__(256) void bw_weight_kernel(const uint16_t* __restrict__ w, int64_t R, int64_t C,
                                                        uint8_t* __restrict__ q, float* __restrict__ s,
                                                        uint8_t* __restrict__ qT) {
  __shared__ uint32_t red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kBwTPitch];
  const int64_t br = blockIdx.y, bcn = blockIdx.x;
  const int t = threadIdx.x;
  const int r = t >> 4, ch = t & 15;
  uint4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t row = br * 128 + r + 16 * i;
    v[i] = load16_nt((const uint4*)(w + row * C + bcn * 128 + ch * 8));                     // read once
    m = max(m, magmax8(v[i]));
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const BwScale sc = bw_scale<POW2>(m);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = r + 16 * i;
    const int64_t row = br * 128 + rr;
    const uint2 o = bw_convert8<POW2>(v[i], sc);
    *(uint2*)(q + row * C + bcn * 128 + ch * 8) = o;
    if (qT) {
      // element (row rr, column 8 ch + b) of the block goes to transposed row 8 ch + b, column rr
      const uint32_t wd[2] = {o.x, o.y};
#pragma unroll
      for (int b = 0; b < 8; ++b) tile[(8 * ch + b) * kBwTPitch + rr] = (uint8_t)(wd[b >> 2] >> (8 * (b & 3)));
    }
  }
  if (t == 0) s[br * (C / 128) + bcn] = sc.s;
  if (qT) {
    __syncthreads();
    // transposed row k (= block column) holds the block's 128 rows: 8 lanes x 16 bytes per row
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 256 + t;
      const int k = idx >> 3, piece = idx & 7;
      const uint4 val = *(const uint4*)(tile + k * kBwTPitch + 16 * piece);
      *(uint4*)(qT + (bcn * 128 + k) * R + br * 128 + 16 * piece) = val;
    }
  }
}

hipError_t launch_bw_act(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, bool pow2, hipStream_t st) {
  int64_t nchunks = R * C / 8;
  if (nchunks == 0) return hipSuccess;
  const int64_t per = (int64_t)kBwActThreads * kBwActUnroll;
  const int64_t blocks = (nchunks + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  if (pow2)
    hipLaunchKernelGGL(bw_act_kernel<true>, grid, dim3(kBwActThreads), 0, st, (const uint4*)x, nchunks, (uint2*)q, s);
  else
    hipLaunchKernelGGL(bw_act_kernel<false>, grid, dim3(kBwActThreads), 0, st, (const uint4*)x, nchunks, (uint2*)q, s);
  return hipGetLastError();
}

hipError_t launch_bw_weight(const uint16_t* w, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT, bool pow2,
                            hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)(C / 128), (unsigned)(R / 128));
  if (pow2)
    hipLaunchKernelGGL(bw_weight_kernel<true>, grid, dim3(256), 0, st, w, R, C, q, s, qT);
  else
    hipLaunchKernelGGL(bw_weight_kernel<false>, grid, dim3(256), 0, st, w, R, C, q, s, qT);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Column-wise blockwise quantiser (the weight-gradient operands of the blockwise recipe): blocks of
// 128 consecutive rows of one column, restarting at every expert's first row, one fp32 scale per
// (column, block).  Output qT [C, ld], sT [C, ld/128]: expert g's rows at columns
// [128 starts[g], 128 starts[g] + m_g), a short last block padded with zero codes, block-columns of
// no expert all zero (codes and scale).
//
// A workgroup (256 lanes) takes one block-column and a window of 128 input columns.  Lane t owns
// columns 2 (t % 64), +1 and rows 32 (t / 64) .. +31 of the block, loaded straight into registers as
// one dword per row (a wave reads 256 contiguous bytes of a row); the column pair's amax is combined
// over the four row quarters through LDS, and the lane's 32 code bytes per column go to an LDS
// output tile that is written out as 128-byte rows of qT.
// ---------------------------------------------------------------------------------------------
constexpr int kBwColPitch = 128 + 16;   // LDS bytes per output (qT) row, padded against bank conflicts
constexpr int kBwMaxGroupsLds = 1024;

template <bool POW2>
__global__ __launch_bounds__(256) void bw_colwise_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                         const int32_t* __restrict__ offs, int G,
                                                         uint8_t* __restrict__ qT, float* __restrict__ sT,
                                                         int64_t ld) {
  __shared__ int32_t starts[kBwMaxGroupsLds + 1];
  __shared__ int32_t rows0[kBwMaxGroupsLds + 1];
  __shared__ __attribute__((aligned(16))) uint8_t outq[128 * kBwColPitch];
  __shared__ uint32_t red[4][64];
  __shared__ int32_t blk[2];

  const int nwin = (int)(C / 128);
  const int win = blockIdx.x % nwin;
  const int bc = blockIdx.x / nwin;
  const int nbc = (int)(ld / 128);
  const int t = threadIdx.x;
  group_block_starts<128>(offs, G, R, starts, rows0);
  __syncthreads();
  if (t == 0) {
    int32_t r0, n;
    block_rows<128>(bc, nbc, G, starts, rows0, r0, n);
    blk[0] = r0;
    blk[1] = n;
  }
  __syncthreads();
  const int r0 = blk[0], n = blk[1];
  const int64_t cbase = (int64_t)win * 128;

  const int cp = t & 63, qq = t >> 6;
  // the lane's column pair in rows 32 qq .. 32 qq + 31 of the block (zeros past n); row addresses are
  // wave-uniform
  uint32_t w[32];
  uint32_t m0 = 0, m1 = 0;
  const int nq = n - 32 * qq;       // rows of this quarter inside the block
  const uint16_t* src = x + ((int64_t)r0 + 32 * qq) * C + cbase + 2 * cp;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    w[r] = r < nq ? __builtin_nontemporal_load((const uint32_t*)(src + (int64_t)r * C)) : 0u;   // read once
    m0 = max(m0, w[r] & 0x7FFFu);
    m1 = max(m1, (w[r] >> 16) & 0x7FFFu);
  }
  red[qq][cp] = m0 | (m1 << 16);
  __syncthreads();
  uint32_t a0 = 0, a1 = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a0 = max(a0, red[k][cp] & 0xFFFFu);
    a1 = max(a1, red[k][cp] >> 16);
  }
  const BwScale sc0 = bw_scale<POW2>(a0), sc1 = bw_scale<POW2>(a1);
  const float s0 = sc0.s, s1 = sc1.s;
  uint32_t o0[8], o1[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    o0[d] = bw_convert4_col<POW2, false>(w + 4 * d, sc0);
    o1[d] = bw_convert4_col<POW2, true>(w + 4 * d, sc1);
  }
  uint4* d0 = (uint4*)(outq + (2 * cp) * kBwColPitch + 32 * qq);
  uint4* d1 = (uint4*)(outq + (2 * cp + 1) * kBwColPitch + 32 * qq);
  d0[0] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  d0[1] = make_uint4(o0[4], o0[5], o0[6], o0[7]);
  d1[0] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  d1[1] = make_uint4(o1[4], o1[5], o1[6], o1[7]);
  if (qq == 0) {
    // a block-column of no expert keeps scale 0; a real all-zero block gets 1
    const int64_t srow = (int64_t)nbc;
    sT[(cbase + 2 * cp) * srow + bc] = n > 0 ? s0 : 0.0f;
    sT[(cbase + 2 * cp + 1) * srow + bc] = n > 0 ? s1 : 0.0f;
  }
  __syncthreads();
  // qT rows cbase .. cbase + 127, bytes [128 bc, 128 bc + 128): 8 lanes x 16 bytes per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + 256 * i;
    const int row = c >> 3, piece = c & 7;
    *(uint4*)(qT + (cbase + row) * ld + (int64_t)bc * 128 + 16 * piece) =
        *(const uint4*)(outq + row * kBwColPitch + 16 * piece);
  }
}

hipError_t launch_bw_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G, uint8_t* qT,
                             float* sT, int64_t ld, bool pow2, hipStream_t st) {
  const int64_t nwg = (ld / 128) * (C / 128);
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (pow2)
    hipLaunchKernelGGL(bw_colwise_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, st, x, R, C, offs, offs ? G : 1, qT,
                       sT, ld);
  else
    hipLaunchKernelGGL(bw_colwise_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, st, x, R, C, offs, offs ? G : 1, qT,
                       sT, ld);
  return hipGetLastError();
}

}  // namespace mxmoe
