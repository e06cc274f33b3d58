// MX quantisers (bf16 -> E4M3 elements + E8M0 shared exponents, 32-element blocks) for gfx950.
//
// Block rule (opensourcebeat.com MXFP8 article, FAQ "What is MXFP8?": 32 elements share one
// exponent; the exponent choice is the OCP MX v1.0 one): e = floor(log2 amax) - 8 clamped to
// [-127, 127], -127 for an all-zero block; scale byte e + 127; element E4M3(v * 2^-e), nearest
// even, saturating at 448.
//
// Both kernels are HBM-bound: 2 bytes read and 1 + 1/32 bytes written per element.
#include "common.h"

namespace mxmoe {

// ---------------------------------------------------------------------------------------------
// Row-wise: one lane owns 16 input bytes (8 bf16, a quarter of a block); the four lanes of a DPP
// quad own one 32-element block and combine their magnitude maxima with two quad permutes.
// A workgroup of 256 lanes covers 4 x 256 consecutive 16-byte chunks (coalesced per step).
// ---------------------------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 4;

__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of the quad ends with the quad's maximum
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
  return m;
}

__device__ __forceinline__ uint32_t mag_max8(const uint4& v) {
  typedef unsigned short v2us __attribute__((ext_vector_type(2)));
  v2us a = __builtin_bit_cast(v2us, v.x & 0x7FFF7FFFu);
  v2us b = __builtin_bit_cast(v2us, v.y & 0x7FFF7FFFu);
  v2us c = __builtin_bit_cast(v2us, v.z & 0x7FFF7FFFu);
  v2us d = __builtin_bit_cast(v2us, v.w & 0x7FFF7FFFu);
  v2us m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

__global__ __launch_bounds__(kRowThreads) void mx_rowwise_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                                  uint2* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t base = (int64_t)blockIdx.x * (kRowThreads * kRowUnroll) + threadIdx.x;
  uint4 v[kRowUnroll];
#pragma unroll
  for (int j = 0; j < kRowUnroll; ++j) {
    int64_t i = base + (int64_t)j * kRowThreads;
    v[j] = i < nchunks ? x[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kRowUnroll; ++j) {
    int64_t i = base + (int64_t)j * kRowThreads;
    // nchunks is a multiple of 4 and quads are 4-aligned, so a quad is wholly in or out of range
    uint32_t m = quad_max(mag_max8(v[j]));
    int e = mx_exponent(m);
    uint32_t cl = mx_clamp_bits(e);
    uint32_t cl2 = cl | (cl << 16);
    float sc = __uint_as_float((uint32_t)(e + 127) << 23);
    uint2 o;
    o.x = cvt4_e4m3(v[j].x, v[j].y, cl2, sc);
    o.y = cvt4_e4m3(v[j].z, v[j].w, cl2, sc);
    if (i < nchunks) {
      q[i] = o;
      if ((threadIdx.x & 3) == 0) s[i >> 2] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_mx_rowwise(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, hipStream_t st) {
  int64_t nchunks = R * C / 8;
  if (nchunks == 0) return hipSuccess;
  int64_t per = (int64_t)kRowThreads * kRowUnroll;
  int64_t blocks = (nchunks + per - 1) / per;
  hipLaunchKernelGGL(mx_rowwise_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, st,
                     (const uint4*)x, nchunks, (uint2*)q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Column-wise (group-blocked, transposed): output column index space is ld; block-column bc
// (32 output columns) holds block b of group g, rows offs[g] + 32b .. min(+32, offs[g+1]).
// A workgroup handles 4 consecutive block-columns x 64 input columns: it stages the (<= 128) input
// rows through LDS, then lane (c, j) reduces column c of block-column j, converts it and writes
// 32 contiguous output bytes; four lanes write 128 contiguous bytes of one output row.
// ---------------------------------------------------------------------------------------------
constexpr int kColThreads = 256;
constexpr int kColCols = 64;                     // input columns per workgroup
constexpr int kColBlk = 4;                       // block-columns per workgroup
constexpr int kColRowStride = 132;               // bytes per staged row (64 bf16 + 4 pad)
constexpr int kColBlkStride = 32 * kColRowStride + 64;   // bytes per staged block (bank offset 16 per block)
constexpr int kMaxGroupsLds = 1024;   // largest G the column-wise quantiser accepts

__device__ __forceinline__ void group_block_starts(const int32_t* offs, int G, int64_t R, int32_t* starts,
                                                   int32_t* rows0) {
  // starts[g] = sum_{h<g} ceil(m_h/32) for g = 0..G (wave 0 scans 64 groups per step); rows0[g] = offs[g]
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
        nb = (int32_t)((m + 31) / 32);
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

__global__ __launch_bounds__(kColThreads) void mx_colwise_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                                 const int32_t* __restrict__ offs, int G,
                                                                 uint8_t* __restrict__ qT, uint8_t* __restrict__ sT,
                                                                 int64_t ld) {
  __shared__ int32_t starts[kMaxGroupsLds + 1];
  __shared__ int32_t rows0[kMaxGroupsLds + 1];
  __shared__ int32_t blk_r0[kColBlk], blk_n[kColBlk];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColBlk * kColBlkStride];

  const int nbc = (int)(ld / 32);
  const int bc0 = blockIdx.x * kColBlk;
  const int64_t c0 = (int64_t)blockIdx.y * kColCols;
  const int t = threadIdx.x;

  group_block_starts(offs, G, R, starts, rows0);
  __syncthreads();
  if (t < kColBlk) {
    int bc = bc0 + t;
    int32_t r0 = 0, n = 0;
    if (bc < nbc && bc < starts[G]) {
      // last group g with starts[g] <= bc (empty groups share their start with the next group)
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (starts[mid] <= bc) lo = mid; else hi = mid - 1;
      }
      int g = lo;
      int b = bc - starts[g];
      int64_t g0 = rows0[g], g1 = rows0[g + 1];
      r0 = (int32_t)(g0 + 32 * (int64_t)b);
      int64_t left = g1 - r0;
      n = (int32_t)(left < 32 ? left : 32);
    }
    blk_r0[t] = r0;
    blk_n[t] = n;
  }
  __syncthreads();

  // stage: chunk id = t + 256 j -> block j, row t/8, 16-byte column chunk t%8
  {
    const int row = t >> 3, ch = t & 7;
#pragma unroll
    for (int j = 0; j < kColBlk; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      int64_t col = c0 + ch * 8;
      if (row < blk_n[j] && col < C) {
        const uint16_t* src = x + (int64_t)(blk_r0[j] + row) * C + col;
        v = *(const uint4*)src;   // C % 32 == 0 and col % 8 == 0: the 8 columns are all in range
      }
      uint8_t* dst = tile + j * kColBlkStride + row * kColRowStride + ch * 16;
      // 132-byte rows are only 4-byte aligned: four dword stores
      ((uint32_t*)dst)[0] = v.x;
      ((uint32_t*)dst)[1] = v.y;
      ((uint32_t*)dst)[2] = v.z;
      ((uint32_t*)dst)[3] = v.w;
    }
  }
  __syncthreads();

  // convert: lane (c = t/4, j = t%4)
  {
    const int c = t >> 2, j = t & 3;
    const int64_t col = c0 + c;
    const int bc = bc0 + j;
    if (col < C && bc < nbc) {
      const uint8_t* src = tile + j * kColBlkStride + c * 2;
      uint32_t w[16];
      uint32_t m = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        uint32_t lo = *(const uint16_t*)(src + (2 * r) * kColRowStride);
        uint32_t hi = *(const uint16_t*)(src + (2 * r + 1) * kColRowStride);
        w[r] = lo | (hi << 16);
        m = max(m, max(lo & 0x7FFFu, hi & 0x7FFFu));
      }
      int e = mx_exponent(m);
      uint32_t cl = mx_clamp_bits(e);
      uint32_t cl2 = cl | (cl << 16);
      float sc = __uint_as_float((uint32_t)(e + 127) << 23);
      uint4 o0, o1;
      o0.x = cvt4_e4m3(w[0], w[1], cl2, sc);
      o0.y = cvt4_e4m3(w[2], w[3], cl2, sc);
      o0.z = cvt4_e4m3(w[4], w[5], cl2, sc);
      o0.w = cvt4_e4m3(w[6], w[7], cl2, sc);
      o1.x = cvt4_e4m3(w[8], w[9], cl2, sc);
      o1.y = cvt4_e4m3(w[10], w[11], cl2, sc);
      o1.z = cvt4_e4m3(w[12], w[13], cl2, sc);
      o1.w = cvt4_e4m3(w[14], w[15], cl2, sc);
      uint4* dst = (uint4*)(qT + col * ld + (int64_t)bc * 32);
      dst[0] = o0;
      dst[1] = o1;
      sT[col * (ld / 32) + bc] = (uint8_t)(blk_n[j] > 0 ? e + 127 : 0);
    }
  }
}

hipError_t launch_mx_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                             uint8_t* qT, uint8_t* sT, int64_t ld, hipStream_t st) {
  if (C == 0 || ld == 0) return hipSuccess;
  int nbc = (int)(ld / 32);
  dim3 grid((unsigned)((nbc + kColBlk - 1) / kColBlk), (unsigned)((C + kColCols - 1) / kColCols));
  hipLaunchKernelGGL(mx_colwise_kernel, grid, dim3(kColThreads), 0, st, x, R, C, offs, offs ? G : 1, qT, sT, ld);
  return hipGetLastError();
}

}  // namespace mxmoe
