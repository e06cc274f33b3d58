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
// A workgroup of 512 lanes covers 2 x 512 consecutive 16-byte chunks (coalesced per step).  Loads
// and stores are non-temporal: every input byte is read once and every output byte written once.
// Measured on MI355X on the expert-shard tensors: 5.9-6.3 TB/s, against 5.0-5.5 TB/s for 256-lane
// workgroups of 4 chunks with ordinary loads and stores.
// ---------------------------------------------------------------------------------------------
constexpr int kRowThreads = 512;
constexpr int kRowUnroll = 2;

// Column-wise output stores: non-temporal in the dual-layout launch (it writes as many bytes as it
// reads), ordinary in the column-wise launch (measured faster there).
template <bool NT>
__device__ __forceinline__ void store16_col(uint4* p, uint4 v) {
  if (NT) __builtin_nontemporal_store(v4u_{v.x, v.y, v.z, v.w}, (v4u_*)p);
  else *p = v;
}
template <bool NT>
__device__ __forceinline__ void store4_col(uint32_t* p, uint32_t v) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
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

// TILED: the scales in the tiled layout [C / 128][R][4] (the four scale bytes of a row's 128-element
// chunk together, the chunk's rows one after another); c32 = C / 32 blocks per row.
template <bool TILED>
__global__ __launch_bounds__(kRowThreads) void mx_rowwise_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                                  uint2* __restrict__ q, uint8_t* __restrict__ s,
                                                                  int64_t R, int64_t c32) {
  const int64_t base = (int64_t)blockIdx.x * (kRowThreads * kRowUnroll) + threadIdx.x;
  uint4 v[kRowUnroll];
#pragma unroll
  for (int j = 0; j < kRowUnroll; ++j) {
    int64_t i = base + (int64_t)j * kRowThreads;
    v[j] = i < nchunks ? load16_nt(x + i) : make_uint4(0, 0, 0, 0);
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
      store8_nt(q + i, o);
      if ((threadIdx.x & 3) == 0) {
        const int64_t blk = i >> 2;
        int64_t off = blk;
        if (TILED) {
          const int64_t r = blk / c32, b = blk - r * c32;
          off = (b >> 2) * (R * 4) + r * 4 + (b & 3);
        }
        s[off] = (uint8_t)(e + 127);
      }
    }
  }
}

hipError_t launch_mx_rowwise(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, bool tiled,
                             hipStream_t st) {
  int64_t nchunks = R * C / 8;
  if (nchunks == 0) return hipSuccess;
  if (tiled && C % 128) return hipErrorInvalidValue;
  int64_t per = (int64_t)kRowThreads * kRowUnroll;
  int64_t blocks = (nchunks + per - 1) / per;
  if (tiled)
    hipLaunchKernelGGL(mx_rowwise_kernel<true>, dim3((unsigned)blocks), dim3(kRowThreads), 0, st,
                       (const uint4*)x, nchunks, (uint2*)q, s, R, C / 32);
  else
    hipLaunchKernelGGL(mx_rowwise_kernel<false>, dim3((unsigned)blocks), dim3(kRowThreads), 0, st,
                       (const uint4*)x, nchunks, (uint2*)q, s, R, C / 32);
  return hipGetLastError();
}

// MXFP4 row-wise: the same lane layout; each lane's 8 elements become 4 bytes (two E2M1 per byte).
__global__ __launch_bounds__(kRowThreads) void mxfp4_rowwise_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                                     uint32_t* __restrict__ q, uint8_t* __restrict__ s) {
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
    const uint32_t m = quad_max(mag_max8(v[j]));
    const int e = mxfp4_exponent(m);
    const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
    const uint32_t o = cvt8_e2m1(v[j].x, v[j].y, v[j].z, v[j].w, sc);
    if (i < nchunks) {
      store4_nt(q + i, o);
      if ((threadIdx.x & 3) == 0) s[i >> 2] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_mxfp4_rowwise(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, hipStream_t st) {
  int64_t nchunks = R * C / 8;
  if (nchunks == 0) return hipSuccess;
  int64_t per = (int64_t)kRowThreads * kRowUnroll;
  int64_t blocks = (nchunks + per - 1) / per;
  hipLaunchKernelGGL(mxfp4_rowwise_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, st, (const uint4*)x, nchunks,
                     (uint32_t*)q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Column-wise (group-blocked, transposed), optionally fused with the row-wise layout.
//
// Output column index space is ld; block-column bc (32 output columns) holds block b of group g,
// rows offs[g] + 32b .. min(+32, offs[g+1]).  A workgroup (4 waves) owns a window of 256 input
// columns and 4 consecutive block-columns, one per wave.  Lane l owns input columns 4l .. 4l + 3 of
// the window and loads its block's 32 rows as 8-byte pieces (a wave reads 512 contiguous bytes of a
// row); the block's first row and row count are wave-uniform, so row addresses are scalar and full
// blocks carry no per-row bounds.
//  * column-wise: each column's amax by packed 16-bit maxima, rows paired by byte permutes and
//    converted; the 32 code bytes of each (column, block) go to an LDS tile of 256 output rows x
//    128 bytes, written out as whole 128-byte row segments, 16 bytes per lane;
//  * row-wise (fused launch): the 8 lanes holding one 32-column block reduce its amax with DPP and
//    convert their 4 elements; codes go straight to q, scale bytes through LDS.
// The dual-layout launch walks whole rows (all column windows of a row run together) and writes
// with non-temporal stores: 4.0-5.4 TB/s on the expert-shard tensors, against 3.8-4.3 TB/s with runs
// of 8 windows and ordinary stores; the column-wise launch keeps runs of 8 windows and ordinary
// stores, which measured faster for it.  Loads are non-temporal.  Measured and dropped on MI355X:
// double-buffered rows (the next block loading while the current one converts), 8 block-columns per
// workgroup, more workgroups per CU, linear reads or linear writes.
// ---------------------------------------------------------------------------------------------
constexpr int kColThreads = 256;
constexpr int kColLaneCols = 4;                    // adjacent input columns per lane (8-byte pieces)
constexpr int kColCols = 64 * kColLaneCols;        // input columns (output rows) per workgroup
constexpr int kColBlk = 4;                         // block-columns per workgroup (one per wave)
constexpr int kColPitch = kColBlk * 32 + 16;       // LDS bytes per output row (padded against bank conflicts)
constexpr int kColWinRun = 8;                      // column windows visited together (grid order)
constexpr int kRowBlks = kColCols / 32;            // row-wise 32-column blocks per window
constexpr int kMaxGroupsLds = 1024;                // largest G the column-wise quantiser accepts

// Magnitude maximum of four bf16 (two dwords), as a bf16 bit pattern.
__device__ __forceinline__ uint32_t mag_max4(uint32_t w0, uint32_t w1) {
  typedef unsigned short v2us __attribute__((ext_vector_type(2)));
  const v2us m = __builtin_elementwise_max(__builtin_bit_cast(v2us, w0 & 0x7FFF7FFFu),
                                           __builtin_bit_cast(v2us, w1 & 0x7FFF7FFFu));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}


typedef uint32_t ColRows __attribute__((ext_vector_type(kColLaneCols / 2)));   // the lane's columns of one row

struct ColArgs {
  const uint16_t* x;
  int64_t R, C;
  int64_t cbase;        // the window's first input column
  const int32_t* row_idx;
  int64_t Rsrc;
  uint8_t* q;
  uint8_t* s;
  uint8_t* qT;
  uint8_t* sT;
  int64_t ld;
  int lane, w, t;
  bool in;              // the lane's columns lie inside the tensor
};

// Issue the loads of one block's rows (r0, n wave-uniform).  Rows past n repeat row n - 1 (zeroed
// after arrival), so no load depends on a per-row branch; an empty block loads nothing.
template <bool GATHER, bool FULLWIN>
__device__ __forceinline__ void col_load(const ColArgs& a, int r0, int n, ColRows (&v)[32]) {
  if (n == 0 || !(FULLWIN || a.in)) {
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = ColRows{};
    return;
  }
  const uint32_t loff = (uint32_t)(2 * kColLaneCols * a.lane);
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    int64_t src_row = (int64_t)r0 + (r < n ? r : n - 1);
    if (GATHER) {
      const int64_t sr = a.row_idx[src_row];
      src_row = sr < 0 ? 0 : (sr >= a.Rsrc ? a.Rsrc - 1 : sr);
    }
    // row base (wave-uniform, scalar registers) plus the lane's 32-bit byte offset
    const char* base = (const char*)(a.x + src_row * a.C + a.cbase);
    // non-temporal: every input byte is read once (measured with the tiled layout: dual launches 4-8%
    // faster on the expert shard, 27-29% on the DeepSeek-V3-16B tensors right after the fp32 dW writes)
    v[r] = __builtin_nontemporal_load((const ColRows*)(base + loff));
  }
}

// Convert the workgroup's 4 blocks (this wave's: rows r0 .. r0 + n of block-column bc0 + w) and write
// them out.
template <bool ROW, bool FULLWIN, bool FP4, bool TILED>
__device__ __forceinline__ void col_group(const ColArgs& a, int r0, int n, int bc0, ColRows (&v)[32],
                                          uint8_t* outq, uint8_t* outs, uint8_t* rsc, const int32_t* g_r0,
                                          const int32_t* g_n) {
  if (n < 32) {
#pragma unroll
    for (int r = 0; r < 32; ++r)
      if (r >= n) v[r] = ColRows{};
  }
  if constexpr (ROW) {
    // The scale byte of row r collects in byte r % 4 of rs[r / 4] (the same in all 8 lanes of a
    // block); lane 8j + i then stores rs[i], rows 4i .. 4i + 3 of block j, to rsc [wave][j][row].
    static_assert(kColLaneCols == 4, "row-wise blocks assume 8 lanes per 32 columns");
    uint32_t rs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint8_t* qrow = a.q + (int64_t)r0 * a.C + a.cbase;   // wave-uniform
    const uint32_t qoff = (uint32_t)(kColLaneCols * a.lane);
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t m = oct_max(mag_max4(v[r][0], v[r][1]));
      const int e = mx_exponent(m);
      const uint32_t cl = mx_clamp_bits(e);
      const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
      const uint32_t o = cvt4_e4m3(v[r][0], v[r][1], cl | (cl << 16), sc);
      rs[r >> 2] |= (uint32_t)(e + 127) << (8 * (r & 3));
      if (r < n && (FULLWIN || a.in)) store4_col<ROW>((uint32_t*)(qrow + r * a.C + qoff), o);
    }
    const int i = a.lane & 7;
    uint32_t mine = rs[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mine = i == k ? rs[k] : mine;
    *(uint32_t*)(rsc + (a.w * kRowBlks + (a.lane >> 3)) * 32 + 4 * i) = mine;
  }
  typedef unsigned short v2us __attribute__((ext_vector_type(2)));
  v2us mx[kColLaneCols / 2];
#pragma unroll
  for (int k = 0; k < kColLaneCols / 2; ++k) mx[k] = v2us{0, 0};
#pragma unroll
  for (int r = 0; r < 32; ++r)
#pragma unroll
    for (int k = 0; k < kColLaneCols / 2; ++k) {
      // the magnitude mask goes through an opaque instruction: as a plain expression the compiler
      // would share it with the row-wise conversion and keep all 64 masked words live
      uint32_t mag;
      asm volatile("v_and_b32 %0, 0x7fff7fff, %1" : "=v"(mag) : "v"(v[r][k]));
      mx[k] = __builtin_elementwise_max(mx[k], __builtin_bit_cast(v2us, mag));
    }
  // LDS bytes per output row: 32 code bytes per block (E4M3), 16 (E2M1, two per byte), plus padding
  constexpr int kPitch = FP4 ? kColBlk * 16 + 16 : kColPitch;
  constexpr int kBlkBytes = FP4 ? 16 : 32;
#pragma unroll
  for (int k = 0; k < kColLaneCols; ++k) {
    const int e = FP4 ? mxfp4_exponent(mx[k >> 1][k & 1]) : mx_exponent(mx[k >> 1][k & 1]);
    const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
    // pair rows of column k through byte permutes (the lower row in the low half)
    const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
    if constexpr (FP4) {
      // rows 8d .. 8d + 7 of column k -> one dword of E2M1 codes
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t pr[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          pr[p] = __builtin_amdgcn_perm(v[8 * d + 2 * p + 1][k >> 1], v[8 * d + 2 * p][k >> 1], sel);
        o[d] = cvt8_e2m1(pr[0], pr[1], pr[2], pr[3], sc);
      }
      *(uint4*)(outq + (kColLaneCols * a.lane + k) * kPitch + kBlkBytes * a.w) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      const uint32_t cl = mx_clamp_bits(e);
      const uint32_t cl2 = cl | (cl << 16);
      // rows 4d..4d+3 of column k
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t p01 = __builtin_amdgcn_perm(v[4 * d + 1][k >> 1], v[4 * d][k >> 1], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(v[4 * d + 3][k >> 1], v[4 * d + 2][k >> 1], sel);
        o[d] = cvt4_e4m3(p01, p23, cl2, sc);
      }
      uint4* dst = (uint4*)(outq + (kColLaneCols * a.lane + k) * kPitch + kBlkBytes * a.w);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    outs[(kColLaneCols * a.lane + k) * kColBlk + a.w] = (uint8_t)(e + 127);   // all-zero (pad) blocks give 0
  }
  // Publish the LDS tiles.  Only LDS needs to be complete: a __syncthreads() would also wait for the
  // row-wise global stores above, putting their write latency on the path.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // write out: output row cbase + rr holds kBlkBytes kColBlk bytes from block-column bc0 (fewer at the
  // right edge of ld), 16 bytes per lane.  Tiled layout ([ld / 128][C][128], E4M3): those 128 bytes are
  // row rr of tile bc0 / 4, so the workgroup's output is one contiguous run of 128 kColCols bytes.
  constexpr int kPieces = kColBlk * kBlkBytes / 16;                // 16-byte pieces per output row
  constexpr int kPiecesPerBlk = kBlkBytes / 16;
  const int64_t nbc = a.ld / 32;
  const int64_t row_bytes = FP4 ? a.ld / 2 : a.ld;
  const int nb = nbc - bc0 < kColBlk ? (int)(nbc - bc0) : kColBlk;  // block-columns inside ld
#pragma unroll
  for (int it = 0; it < kColCols * kPieces / kColThreads; ++it) {
    const int idx = it * kColThreads + a.t;
    const int rr = idx / kPieces, piece = idx % kPieces;
    const int64_t c = a.cbase + rr;
    if ((FULLWIN || c < a.C) && (piece / kPiecesPerBlk) < nb) {
      const uint4 val = *(const uint4*)(outq + rr * kPitch + 16 * piece);
      const int64_t off = TILED ? (int64_t)(bc0 / kColBlk) * a.C * (kColBlk * kBlkBytes) + c * (kColBlk * kBlkBytes)
                                : c * row_bytes + (int64_t)bc0 * kBlkBytes;
      store16_col<ROW>((uint4*)(a.qT + off + 16 * piece), val);
    }
  }
  if (TILED || (nb == kColBlk && (nbc & 3) == 0)) {
    // the 4 scale bytes of a column are one aligned dword of its sT row; tiled layout
    // ([ld / 128][C][4], ld % 128 == 0, so nb == 4): the workgroup's dwords are one contiguous run
    for (int rr = a.t; rr < kColCols; rr += kColThreads) {
      const int64_t c = a.cbase + rr;
      const int64_t off = TILED ? (int64_t)(bc0 / kColBlk) * a.C * kColBlk + c * kColBlk : c * nbc + bc0;
      if (FULLWIN || c < a.C) *(uint32_t*)(a.sT + off) = *(const uint32_t*)(outs + rr * kColBlk);
    }
  } else {
    for (int idx = a.t; idx < kColCols * kColBlk; idx += kColThreads) {
      const int rr = idx / kColBlk, bb = idx % kColBlk;
      const int64_t c = a.cbase + rr;
      if ((FULLWIN || c < a.C) && bb < nb) a.sT[c * nbc + bc0 + bb] = outs[idx];
    }
  }
  if constexpr (ROW) {
    // row-wise scales: the window's (up to) 8 bytes of each row of the 4 blocks, one lane per row
    const int64_t c32 = a.C / 32;
    const int nrb = FULLWIN ? kRowBlks : (int)((a.C - a.cbase) / 32 < kRowBlks ? (a.C - a.cbase) / 32 : kRowBlks);
    for (int idx = a.t; idx < kColBlk * 32; idx += kColThreads) {
      const int wb = idx >> 5, r = idx & 31;
      if (r < g_n[wb]) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) lo |= (uint32_t)rsc[(wb * kRowBlks + j) * 32 + r] << (8 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) hi |= (uint32_t)rsc[(wb * kRowBlks + 4 + j) * 32 + r] << (8 * j);
        const int64_t row = (int64_t)g_r0[wb] + r;
        if (TILED) {
          // tiled scales [C / 128][R][4] (C % 128 == 0, so nrb is 4 or 8): one dword per 128-column
          // chunk, the chunk's rows one after another
          uint8_t* dst = a.s + (a.cbase / 128) * (a.R * 4) + row * 4;
          *(uint32_t*)dst = lo;
          if (nrb > 4) *(uint32_t*)(dst + a.R * 4) = hi;
        } else {
          uint8_t* dst = a.s + row * c32 + a.cbase / 32;
          if (nrb == kRowBlks && ((uintptr_t)dst & 7) == 0) {
            *(uint2*)dst = make_uint2(lo, hi);
          } else {
            for (int j = 0; j < nrb; ++j) dst[j] = (uint8_t)((j < 4 ? lo : hi) >> (8 * (j & 3)));
          }
        }
      }
    }
  }
}

// ROW: the same launch also writes the row-wise layout (q [R, C], s [R, C/32]) of every row it
// reads; each routed row lies in exactly one block-column, so it is written once.  GATHER: routed
// row r is read from source row row_idx[r] (clamped into [0, Rsrc)).  FULLWIN: C % 256 == 0, so every
// window lies inside the tensor.
template <bool ROW, bool GATHER, bool FULLWIN, bool FP4, bool TILED>
__global__ __launch_bounds__(kColThreads) void mx_colwise_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                                 const int32_t* __restrict__ offs, int G,
                                                                 uint8_t* __restrict__ qT, uint8_t* __restrict__ sT,
                                                                 int64_t ld, uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ s,
                                                                 const int32_t* __restrict__ row_idx, int64_t Rsrc) {
  // The group table (starts, rows0) is dead once the block rows are known, so it shares its LDS with
  // the output tile: 39 KiB per workgroup, four workgroups per CU.
  __shared__ __attribute__((aligned(16))) uint8_t outq[kColCols * kColPitch];
  static_assert(2 * (kMaxGroupsLds + 1) * sizeof(int32_t) <= sizeof(outq), "group table must fit in the output tile");
  int32_t* starts = (int32_t*)outq;
  int32_t* rows0 = starts + (kMaxGroupsLds + 1);
  __shared__ int32_t blk_r0[kColBlk], blk_n[kColBlk];
  __shared__ __attribute__((aligned(16))) uint8_t outs[kColCols * kColBlk];
  __shared__ __attribute__((aligned(8))) uint8_t rsc[ROW ? kColBlk * 32 * kRowBlks : 8];

  const int nbc = (int)(ld / 32);
  // workgroup -> (column window, block-column group), 8 adjacent column windows fastest: the
  // workgroups in flight together read a compact region (whole 4 KiB row pieces) and write runs of
  // neighbouring block-columns
  const int nwin = (int)((C + kColCols - 1) / kColCols);
  const int ngrp = (nbc + kColBlk - 1) / kColBlk;
  // dual layout: a run spans the whole row, so the row-wise codes of consecutive workgroups form
  // whole output rows
  const int run = ROW ? nwin : kColWinRun;
  const int cw = nwin < run ? nwin : run;
  const int chunk = blockIdx.x / (cw * ngrp);
  const int inchunk = blockIdx.x - chunk * cw * ngrp;
  const int cw_here = (nwin - chunk * cw) < cw ? (nwin - chunk * cw) : cw;
  const int win = chunk * cw + inchunk % cw_here;
  const int bc0 = (inchunk / cw_here) * kColBlk;
  const int t = threadIdx.x;
  if (offs) {
    group_block_starts<32>(offs, G, R, starts, rows0);
    __syncthreads();
  }
  if (t < kColBlk) {
    const int bc = bc0 + t;
    int32_t r0 = 0, n = 0;
    if (offs) {
      block_rows<32>(bc, nbc, G, starts, rows0, r0, n);
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

  ColArgs a;
  a.x = x; a.R = R; a.C = C; a.cbase = (int64_t)win * kColCols; a.row_idx = row_idx; a.Rsrc = Rsrc;
  a.q = q; a.s = s; a.qT = qT; a.sT = sT; a.ld = ld;
  a.t = t; a.w = t >> 6; a.lane = t & 63;
  a.in = a.cbase + kColLaneCols * a.lane < C;   // C % 32 == 0: all or none of the lane's columns
  const int r0 = __builtin_amdgcn_readfirstlane(blk_r0[a.w]);
  const int n = __builtin_amdgcn_readfirstlane(blk_n[a.w]);
  ColRows v[32];
  col_load<GATHER, FULLWIN>(a, r0, n, v);
  col_group<ROW, FULLWIN, FP4, TILED>(a, r0, n, bc0, v, outq, outs, rsc, blk_r0, blk_n);
}

static int64_t colwise_grid(int64_t C, int64_t ld) {
  return ((ld / 32 + kColBlk - 1) / kColBlk) * ((C + kColCols - 1) / kColCols);
}

template <bool ROW, bool GATHER, bool FP4 = false, bool TILED = false>
static void launch_col(bool fullwin, int64_t nwg, hipStream_t st, const uint16_t* x, int64_t R, int64_t C,
                       const int32_t* offs, int32_t G, uint8_t* qT, uint8_t* sT, int64_t ld, uint8_t* q, uint8_t* s,
                       const int32_t* row_idx, int64_t Rsrc) {
  static_assert(!(TILED && FP4), "the tiled layout holds E4M3 codes");
  if (fullwin)
    hipLaunchKernelGGL((mx_colwise_kernel<ROW, GATHER, true, FP4, TILED>), dim3((unsigned)nwg), dim3(kColThreads), 0,
                       st, x, R, C, offs, G, qT, sT, ld, q, s, row_idx, Rsrc);
  else
    hipLaunchKernelGGL((mx_colwise_kernel<ROW, GATHER, false, FP4, TILED>), dim3((unsigned)nwg), dim3(kColThreads), 0,
                       st, x, R, C, offs, G, qT, sT, ld, q, s, row_idx, Rsrc);
}

hipError_t launch_mx_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                             uint8_t* qT, uint8_t* sT, int64_t ld, bool tiled, hipStream_t st) {
  if (C == 0 || ld == 0) return hipSuccess;
  if (tiled && ld % 128) return hipErrorInvalidValue;
  const int64_t nwg = colwise_grid(C, ld);
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (tiled)
    launch_col<false, false, false, true>(C % kColCols == 0, nwg, st, x, R, C, offs, offs ? G : 1, qT, sT, ld, nullptr,
                                          nullptr, nullptr, (int64_t)0);
  else
    launch_col<false, false>(C % kColCols == 0, nwg, st, x, R, C, offs, offs ? G : 1, qT, sT, ld, nullptr, nullptr,
                             nullptr, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_mxfp4_colwise(const uint16_t* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                                uint8_t* qT, uint8_t* sT, int64_t ld, hipStream_t st) {
  if (C == 0 || ld == 0) return hipSuccess;
  const int64_t nwg = colwise_grid(C, ld);
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_col<false, false, true>(C % kColCols == 0, nwg, st, x, R, C, offs, offs ? G : 1, qT, sT, ld, nullptr,
                                 nullptr, nullptr, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_mx_dual(const uint16_t* x, int64_t R, int64_t C, const int32_t* row_idx, int64_t Rsrc,
                          const int32_t* offs, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT, int64_t ld,
                          bool tiled, hipStream_t st) {
  if (C == 0 || ld == 0) return hipSuccess;
  if (tiled && (ld % 128 || C % 128)) return hipErrorInvalidValue;
  const int64_t nwg = colwise_grid(C, ld);
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool fw = C % kColCols == 0;
  const int32_t g = offs ? G : 1;
  if (row_idx && tiled) launch_col<true, true, false, true>(fw, nwg, st, x, R, C, offs, g, qT, sT, ld, q, s, row_idx, Rsrc);
  else if (row_idx) launch_col<true, true>(fw, nwg, st, x, R, C, offs, g, qT, sT, ld, q, s, row_idx, Rsrc);
  else if (tiled) launch_col<true, false, false, true>(fw, nwg, st, x, R, C, offs, g, qT, sT, ld, q, s, nullptr, R);
  else launch_col<true, false>(fw, nwg, st, x, R, C, offs, g, qT, sT, ld, q, s, nullptr, R);
  return hipGetLastError();
}

}  // namespace mxmoe
