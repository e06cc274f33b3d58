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
// A workgroup handles 4 W consecutive block-columns x 64 P input columns (W block-columns per wave,
// P adjacent columns per lane).  Lane l of wave w owns input columns P l .. P l + P - 1 of the tile
// and, for each of the wave's block-columns, loads the block's (<= 32) rows as 2P-byte pieces (a
// wave reads 128 P contiguous bytes of a row), takes each column's amax with packed 16-bit maxima,
// pairs rows with byte permutes and converts them.  The 32 code bytes of each (column, block) go to
// an LDS tile of 64 P output rows x 128 W bytes, which the workgroup then writes out as whole row
// segments, 16 bytes per lane.
// ---------------------------------------------------------------------------------------------
#ifndef MXMOE_COL_LANE_COLS
#define MXMOE_COL_LANE_COLS 4
#endif
#ifndef MXMOE_COL_WAVE_BLKS
#define MXMOE_COL_WAVE_BLKS 1
#endif
constexpr int kColThreads = 256;
constexpr int kColLaneCols = MXMOE_COL_LANE_COLS;  // adjacent input columns per lane (4: 8-byte pieces)
constexpr int kColWaveBlks = MXMOE_COL_WAVE_BLKS;  // block-columns per wave
constexpr int kColCols = 64 * kColLaneCols;        // input columns (output rows) per workgroup
constexpr int kColBlk = 4 * kColWaveBlks;          // consecutive block-columns per workgroup
constexpr int kColPitch = kColBlk * 32 + 16;       // LDS bytes per output row (padded against bank conflicts)
constexpr int kColWinRun = 8;                      // column windows visited together (grid order)
constexpr int kMaxGroupsLds = 1024;              // largest G the column-wise quantiser accepts

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
  __shared__ __attribute__((aligned(16))) uint8_t outq[kColCols * kColPitch];
  __shared__ uint8_t outs[kColCols * kColBlk];

  const int nbc = (int)(ld / 32);
  // workgroup -> (column window, block-column group), 8 adjacent column windows fastest: the
  // workgroups in flight together read a compact region (whole 4 KiB row pieces) and write runs of
  // neighbouring block-columns
  const int nwin = (int)((C + kColCols - 1) / kColCols);
  const int ngrp = (nbc + kColBlk - 1) / kColBlk;
  const int cw = nwin < kColWinRun ? nwin : kColWinRun;
  const int chunk = blockIdx.x / (cw * ngrp);
  const int inchunk = blockIdx.x - chunk * cw * ngrp;
  const int cw_here = (nwin - chunk * cw) < cw ? (nwin - chunk * cw) : cw;
  const int win = chunk * cw + inchunk % cw_here;
  const int bc0 = (inchunk / cw_here) * kColBlk;
  const int t = threadIdx.x;
  if (offs) {
    group_block_starts(offs, G, R, starts, rows0);
    __syncthreads();
  }
  if (t < kColBlk) {
    const int bc = bc0 + t;
    int32_t r0 = 0, n = 0;
    if (offs) {
      if (bc < nbc && bc < starts[G]) {
        // last group g with starts[g] <= bc (empty groups share their start with the next group)
        int lo = 0, hi = G - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (starts[mid] <= bc) lo = mid; else hi = mid - 1;
        }
        const int64_t g0 = rows0[lo], g1 = rows0[lo + 1];
        r0 = (int32_t)(g0 + 32 * (int64_t)(bc - starts[lo]));
        const int64_t left = g1 - r0;
        n = (int32_t)(left < 32 ? left : 32);
      }
    } else if (bc < nbc) {
      // one group of R rows
      r0 = 32 * bc;
      const int64_t left = R - r0;
      n = (int32_t)(left < 0 ? 0 : (left < 32 ? left : 32));
    }
    blk_r0[t] = r0;
    blk_n[t] = n;
  }
  __syncthreads();

  const int64_t cbase = (int64_t)win * kColCols;
  const int w = t >> 6, lane = t & 63;
  typedef uint32_t vcols __attribute__((ext_vector_type(kColLaneCols / 2)));   // the lane's columns of one row
  for (int wb = 0; wb < kColWaveBlks; ++wb) {
    // block-column bc0 + bl of the workgroup, columns cbase + kColLaneCols * lane ..
    const int bl = w * kColWaveBlks + wb;
    const int n = blk_n[bl];
    const int64_t c = cbase + kColLaneCols * lane;
    vcols v[32];
    if (c < C) {   // C % 32 == 0 and c % kColLaneCols == 0: the lane's columns are all in range
      const uint16_t* src = x + (int64_t)blk_r0[bl] * C + c;
#pragma unroll
      for (int r = 0; r < 32; ++r) v[r] = r < n ? *(const vcols*)(src + r * C) : vcols{};
    } else {
#pragma unroll
      for (int r = 0; r < 32; ++r) v[r] = vcols{};
    }
    typedef unsigned short v2us __attribute__((ext_vector_type(2)));
    v2us mx[kColLaneCols / 2];
#pragma unroll
    for (int q = 0; q < kColLaneCols / 2; ++q) mx[q] = v2us{0, 0};
#pragma unroll
    for (int r = 0; r < 32; ++r)
#pragma unroll
      for (int q = 0; q < kColLaneCols / 2; ++q)
        mx[q] = __builtin_elementwise_max(mx[q], __builtin_bit_cast(v2us, v[r][q] & 0x7FFF7FFFu));
#pragma unroll
    for (int k = 0; k < kColLaneCols; ++k) {
      const int e = mx_exponent(mx[k >> 1][k & 1]);
      const uint32_t cl = mx_clamp_bits(e);
      const uint32_t cl2 = cl | (cl << 16);
      const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
      // rows 4d..4d+3 of column k: pair rows through byte permutes (row a in the low half)
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t p01 = __builtin_amdgcn_perm(v[4 * d + 1][k >> 1], v[4 * d][k >> 1], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(v[4 * d + 3][k >> 1], v[4 * d + 2][k >> 1], sel);
        o[d] = cvt4_e4m3(p01, p23, cl2, sc);
      }
      uint4* dst = (uint4*)(outq + (kColLaneCols * lane + k) * kColPitch + 32 * bl);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      outs[(kColLaneCols * lane + k) * kColBlk + bl] = (uint8_t)(e + 127);   // all-zero (pad) blocks give 0
    }
  }
  __syncthreads();

  // write out: output row cbase + rr holds 32 kColBlk bytes from column 32 bc0 (fewer at the right
  // edge of ld), 16 bytes per lane
  constexpr int kPieces = kColBlk * 2;                             // 16-byte pieces per output row
  const int nb = nbc - bc0 < kColBlk ? nbc - bc0 : kColBlk;       // block-columns inside ld
  const int64_t lds32 = ld / 32;
#pragma unroll
  for (int it = 0; it < kColCols * kPieces / kColThreads; ++it) {
    const int idx = it * kColThreads + t;
    const int rr = idx / kPieces, piece = idx % kPieces;
    const int64_t c = cbase + rr;
    if (c < C && (piece >> 1) < nb) {
      const uint4 val = *(const uint4*)(outq + rr * kColPitch + 16 * piece);
      *(uint4*)(qT + c * ld + (int64_t)bc0 * 32 + 16 * piece) = val;
    }
  }
  for (int idx = t; idx < kColCols * kColBlk; idx += kColThreads) {
    const int rr = idx / kColBlk, b = idx % kColBlk;
    const int64_t c = cbase + rr;
    if (c < C && b < nb) sT[c * lds32 + bc0 + b] = outs[idx];
  }
}

hipError_t launch_mx_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                             uint8_t* qT, uint8_t* sT, int64_t ld, hipStream_t st) {
  if (C == 0 || ld == 0) return hipSuccess;
  int nbc = (int)(ld / 32);
  const int64_t nwg = (int64_t)((nbc + kColBlk - 1) / kColBlk) * ((C + kColCols - 1) / kColCols);
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  hipLaunchKernelGGL(mx_colwise_kernel, grid, dim3(kColThreads), 0, st, x, R, C, offs, offs ? G : 1, qT, sT, ld);
  return hipGetLastError();
}

}  // namespace mxmoe
