// Device helpers shared by the grouped GEMM kernels of gfx950 (MX and blockwise FP8): the tile list of
// a dropless grouped launch built from the device-resident group offsets, direct-to-LDS loads, the
// stage barrier and the exact E4M3 -> bf16 widening.
#pragma once

#include "common.h"

namespace mxmoe {

constexpr int kMaxG = 1024;                      // largest expert count of a launch
constexpr int kXcd = 8;                          // workgroups go round-robin over the 8 XCDs
constexpr int kGroupM = 4;                       // A tiles per raster column inside an expert
// Consecutive tiles one XCD takes per visit.  Forward and dgrad: 16, so that (with the raster above)
// the 32 tiles an XCD runs at once span about 8 A and 4 B tiles, 12 operand panels, where chunks of 8
// gave 16 A and 2 B tiles (18 panels, every A panel fetched by all eight XCDs).  Weight gradient: 8
// (its largest-expert-first list ran 4% slower with 16).
constexpr int chunk_tiles(int mode) { return mode == kWgrad ? 8 : 16; }
constexpr int kLptMaxG = 256;                    // wgrad orders experts by size up to this G

struct GroupTile {
  int g, mt, nt;
  int64_t row0;   // forward / dgrad: first A row of the tile
  int rows;       // forward / dgrad: valid A rows of the tile
  int64_t col0;   // wgrad, gated forward: first column of the expert in the column-wise layout
  int nblk;       // wgrad: blocks (of the column-wise layout) in the expert's contraction
  int64_t col_end;  // gated forward: columns of the column-wise layout holding blocks (all experts)
};

__device__ __forceinline__ int cdiv(int64_t a, int b) { return (int)((a + b - 1) / b); }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Tile list of the launch and this workgroup's tile.  Scratch arrays live at the start of the LDS
// (before the first operand load overwrites them).  Returns false when the workgroup has no tile.
// Tiles are TBM A rows x TBN B rows; TNT threads.  CB: also the first CBLK-block of each expert in the
// column-wise layout (wgrad; the gated forward's column-wise H), whose blocks are CBLK rows.
// PARTIAL_LAST (forward, dgrad): the experts' full row tiles come first, in expert order, and their
// partial last row tiles after them, the ones with the most rows first (for G <= kLptMaxG), so that
// the launch's last round holds the tiles with the fewest rows (cheaper where idle waves skip their
// MFMAs).
template <int MODE, bool CB, int TBM, int TBN, int TNT, int CBLK, bool PARTIAL_LAST = false>
__device__ bool decode_grouped_tile(const GemmArgs& p, char* lds, GroupTile& t) {
  int32_t* s_rs = (int32_t*)lds;             // clamped offsets [G+1]
  int32_t* s_pre = s_rs + (kMaxG + 1);       // tile prefix over the processing order [G+1]
  int32_t* s_cb = s_pre + (kMaxG + 1);       // wgrad: first 32-block of each expert [G+1]
  int32_t* s_ord = s_cb + (kMaxG + 1);       // processing order [G] (PARTIAL_LAST: of the partial tiles)
  int32_t* s_pre2 = s_ord + kMaxG;           // PARTIAL_LAST: prefix of the partial tiles [G+1]
  constexpr bool kSplit = PARTIAL_LAST && MODE != kWgrad;
  const int G = p.G;
  const int tid = threadIdx.x;
  const int64_t M = p.M;
  for (int g = tid; g <= G; g += TNT) s_rs[g] = (int32_t)clamp_off(p.offs[g], M);
  __syncthreads();
  // wgrad: experts by size; split forward / dgrad: the partial tiles by their rows (m_g mod TBM, 0 for
  // none); largest first, ties by index
  const bool lpt = (MODE == kWgrad || kSplit) && G <= kLptMaxG;
  auto key = [&](int g) {
    const int m = max(s_rs[g + 1] - s_rs[g], 0);
    return kSplit ? m % TBM : m;
  };
  if (lpt) {
    // the rank of expert g: eight consecutive lanes count the experts h = part, part + 8, ... that go
    // before g, and their counts are summed across the eight lanes
    static_assert(TNT % 64 == 0, "whole waves");
    for (int idx = tid; idx < 8 * G; idx += TNT) {
      const int g = idx >> 3, part = idx & 7;
      const int mg = key(g);
      int pos = 0;
      for (int h = part; h < G; h += 8) {
        const int mh = key(h);
        pos += (mh > mg) || (mh == mg && h < g);
      }
      pos += __shfl_xor(pos, 1, 64);
      pos += __shfl_xor(pos, 2, 64);
      pos += __shfl_xor(pos, 4, 64);
      if (part == 0) s_ord[pos] = g;
    }
  } else {
    for (int g = tid; g < G; g += TNT) s_ord[g] = g;
  }
  __syncthreads();
  const int ntc = cdiv(MODE == kFwd ? p.N : p.K, TBN);
  const int mtc_w = cdiv(p.N, TBM);
  const int lane = tid & 63;
  // prefix sums, one wave each: the tiles (full row tiles when split) over the processing order (expert
  // order when split), the blocks of each expert (CB), the partial tiles over s_ord (split)
  const int wv = tid >> 6;
  const bool cb_wave = CB && wv == 1;
  const bool p2_wave = kSplit && wv == 2;
  if (wv == 0 || cb_wave || p2_wave) {
    int carry = 0;
    for (int base = 0; base < G; base += 64) {
      const int q = base + lane;
      int c = 0;
      if (q < G) {
        if (wv == 0) {
          const int g = kSplit ? q : s_ord[q];
          const int mg = max(s_rs[g + 1] - s_rs[g], 0);
          if (MODE == kWgrad) c = mtc_w * ntc;
          else c = (kSplit ? mg / TBM : cdiv(mg, TBM)) * ntc;
        } else if (cb_wave) {
          c = cdiv(max(s_rs[q + 1] - s_rs[q], 0), CBLK);
        } else {
          const int g = s_ord[q];
          c = (max(s_rs[g + 1] - s_rs[g], 0) % TBM ? 1 : 0) * ntc;
        }
      }
      int incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      int32_t* dst = wv == 0 ? s_pre : (cb_wave ? s_cb : s_pre2);
      if (q < G) dst[q] = carry + incl - c;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) (wv == 0 ? s_pre : (cb_wave ? s_cb : s_pre2))[G] = carry;
  }
  __syncthreads();

  // workgroup -> logical tile: chunks of kChunk consecutive tiles per XCD visit
  constexpr int kChunk = chunk_tiles(MODE);
  const int b = blockIdx.x;
  const int x = b % kXcd, q = b / kXcd;
  const int lt_all = ((q / kChunk) * kXcd + x) * kChunk + (q % kChunk);
  const int n_full = s_pre[G];
  if (lt_all >= n_full + (kSplit ? s_pre2[G] : 0)) return false;
  int g, mt, nt, mtc;
  if (kSplit && lt_all >= n_full) {
    // a partial last row tile: expert by the partial-tile prefix, then its column tile
    const int lt2 = lt_all - n_full;
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre2[mid] <= lt2) lo = mid; else hi = mid - 1;
    }
    g = s_ord[lo];
    mtc = max(s_rs[g + 1] - s_rs[g], 0) / TBM;      // full row tiles before it
    mt = mtc;
    nt = lt2 - s_pre2[lo];
  } else {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= lt_all) lo = mid; else hi = mid - 1;
    }
    g = kSplit ? lo : s_ord[lo];
    const int lt = lt_all - s_pre[lo];
    const int m_g = max(s_rs[g + 1] - s_rs[g], 0);
    mtc = MODE == kWgrad ? mtc_w : (kSplit ? m_g / TBM : cdiv(m_g, TBM));
    const int span = kGroupM * ntc;
    const int sg = lt / span;
    const int fm = sg * kGroupM;
    const int gsz = min(mtc - fm, kGroupM);
    const int r = lt - sg * span;
    mt = fm + r % gsz;
    nt = r / gsz;
  }
  const int m_g = max(s_rs[g + 1] - s_rs[g], 0);
  t.g = g;
  t.mt = mt;
  t.nt = nt;
  t.row0 = s_rs[g] + (int64_t)t.mt * TBM;
  t.rows = (int)min((int64_t)TBM, (int64_t)s_rs[g + 1] - t.row0);
  t.col0 = CB ? CBLK * (int64_t)s_cb[g] : 0;
  t.col_end = CB ? CBLK * (int64_t)s_cb[G] : 0;
  t.nblk = cdiv(m_g, CBLK);
  if (MODE == kWgrad) {
    // offsets that are not monotone could place an expert past the leading dimension: clip
    const int64_t ld_el = p.ld_cols;
    const int64_t room = ld_el > t.col0 ? (ld_el - t.col0) / CBLK : 0;
    if (t.nblk > room) t.nblk = (int)room;
  }
  return true;
}

// Store a wave's accumulator tile as whole row pieces.  The tile is NI x NJ fragments of 32 x 32 in
// the layout of an MFMA that takes the B fragment first: lane l holds tile row 32 i + l % 32 and, per
// group q of four registers, columns 32 j + 8 q + 4 (l / 32) .. + 3.  RPP fragment rows (32 RPP rows) at
// a time go to the wave's own LDS region `reg` (>= 32 RPP (128 NJ + 16) bytes, 16-byte aligned), as fp32
// or bf16, and leave 16 bytes per lane: an instruction writes 4 rows x 128 NJ bytes (fp32) or 8 rows x
// 64 NJ bytes (bf16), where stores straight from the accumulators write 32 rows x 16 or 32 bytes.
// Output element (tile row r, tile column c) is out[(out_row0 + r0 + r) * nout + col0 + c0 + c]; rows at
// or past row_lim and column groups at or past col_lim are not written (col_lim a multiple of 8).  The
// region must be free (the caller's barrier); a wave's own LDS accesses stay in order, so the passes
// and the write and read of a pass need no barrier.  A pass reads all its pieces from LDS before it
// stores any (unrolled), so the LDS latency is paid once per pass rather than once per piece.
template <int NI, int NJ, int RPP, bool BF16, typename Acc>
__device__ __forceinline__ void store_tile_rows_as(const Acc (&acc)[NI][NJ], char* reg, void* out, int64_t out_row0,
                                                   int64_t nout, int64_t col0, int r0, int c0, int row_lim,
                                                   int col_lim) {
  static_assert(NI % RPP == 0, "passes of RPP fragment rows");
  constexpr int kPitch = BF16 ? 64 * NJ + 16 : 128 * NJ + 16;    // bytes per staged row
  constexpr int kCpr = BF16 ? 4 * NJ : 8 * NJ;                    // 16-byte pieces per staged row
  constexpr int kPieces = 32 * RPP * kCpr / 64;                   // pieces per lane and pass
  static_assert(32 * RPP * kCpr % 64 == 0, "whole pieces per lane");
  const int lane = threadIdx.x & 63, h = lane >> 5;
#pragma unroll
  for (int pass = 0; pass < NI / RPP; ++pass) {
#pragma unroll
    for (int ii = 0; ii < RPP; ++ii) {
      const int i = RPP * pass + ii;
      const int r = (lane & 31) + 32 * ii;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 32 * j + 8 * q + 4 * h;
          const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
          const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          if constexpr (BF16)
            *(uint2*)(reg + r * kPitch + 2 * c) = make_uint2(f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16),
                                                             f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16));
          else
            *(float4*)(reg + r * kPitch + 4 * c) = make_float4(v0, v1, v2, v3);
        }
    }
    uint4 v[kPieces];
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int k = lane + 64 * it;
      v[it] = *(const uint4*)(reg + (k / kCpr) * kPitch + 16 * (k % kCpr));
    }
    // Left alone, the compiler sinks each read into the row test of its store, which then waits out the
    // LDS latency once per piece.  An empty asm that takes every piece keeps the reads ahead of the stores.
#pragma unroll
    for (int it = 0; it < kPieces; ++it) asm volatile("" : "+v"(v[it].x), "+v"(v[it].y), "+v"(v[it].z), "+v"(v[it].w));
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int k = lane + 64 * it;
      const int tr = r0 + 32 * RPP * pass + k / kCpr;               // tile row
      const int tc = c0 + (k % kCpr) * (BF16 ? 8 : 4);             // tile column of the piece's first element
      if (tr >= row_lim || tc >= col_lim) continue;
      const int64_t idx = (out_row0 + tr) * nout + col0 + tc;
      if constexpr (BF16) *(uint4*)((uint16_t*)out + idx) = v[it];
      else *(uint4*)((float*)out + idx) = v[it];
    }
  }
}

// The same with the output type chosen at run time (a kernel argument: uniform).
template <int NI, int NJ, int RPP, typename Acc>
__device__ __forceinline__ void store_tile_rows(const Acc (&acc)[NI][NJ], char* reg, bool bf16, void* out,
                                                int64_t out_row0, int64_t nout, int64_t col0, int r0, int c0,
                                                int row_lim, int col_lim) {
  if (bf16) store_tile_rows_as<NI, NJ, RPP, true>(acc, reg, out, out_row0, nout, col0, r0, c0, row_lim, col_lim);
  else store_tile_rows_as<NI, NJ, RPP, false>(acc, reg, out, out_row0, nout, col0, r0, c0, row_lim, col_lim);
}

// Eight E4M3 bytes -> eight bf16 multiplied by 2^(e-127), e the E8M0 byte whose bits sit in the
// exponent field of `scale`; exact for every product the GEMMs form.
__device__ __forceinline__ v8bf widen8(uint32_t w0, uint32_t w1, float scale) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float e8m0_as_scale(uint32_t word, int b) {
  return __uint_as_float(((word >> (8 * b)) & 0xFFu) << 23);
}

// Direct global -> LDS loads.  Lane l writes its bytes at LDS address m0 + size * l, m0 being the
// wave-uniform base.  Issued from inline assembly so that the compiler does not treat them as LDS
// stores it must wait for before every later LDS read: the kernel orders them itself (stage_barrier).
// Nothing else in these kernels uses m0.
__device__ __forceinline__ uint32_t lds_addr(const char* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ void dma16(const uint8_t* g, const char* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))), "v"(g) : "memory", "m0");
}
// The same load addressed as a wave-uniform 64-bit base (scalar registers) plus a 32-bit lane offset:
// per stage only the base moves (scalar adds), the lane offsets are formed once per tile.
__device__ __forceinline__ void dma16s(uint32_t off, const uint8_t* base, const char* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))), "v"(off), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* g, const char* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base))), "v"(g) : "memory", "m0");
}

// Wait for this wave's outstanding loads and LDS operations, then the workgroup barrier.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mxmoe
