// Blockwise-FP8 dropless grouped GEMM for MoE experts on gfx950 (the DeepSeek-V3 fine-grained recipe).
//
// aifind.ru, "DeepSeek-V3: a revolutionary high-performance language model with low training cost", section
// "Low-precision training: FP8 Framework", captions (a) and (b): activations carry an fp32 scale per 1x128
// tile, weights per 128x128 block, and the FP8 products are summed over each 128-element slice of the
// contraction before that partial is promoted, i.e. multiplied by its two scales and added to a
// full-precision accumulator.  All experts run in one launch, each on its real number of rows (iitak.ru,
// "NVIDIA sped up training of mixture-of-experts models on JAX tenfold": no capacity padding, no dropped
// tokens): the launch enumerates the 128x128 output tiles of all experts from the device-resident group
// offsets, so an expert with no rows contributes no tile (forward / dgrad) and one with a handful of rows
// one partial tile.
//
// Generic form computed by one workgroup (tile (mt, nt) of expert g), promoted per 128-slice kb:
//   out[i, j] = sum_kb sA(i, kb) sB(j, kb) sum_{t in kb} A[row_a(i), col0_a + t] * B[row_b(j), col0_b + t]
// where
//   forward: A = X rows of expert g, B = W_g rows, sA = the 1x128 tile scale, sB = the 128x128 block scale
//   dgrad:   A = dY rows of expert g (1x128 tiles along N), B = the transposed weight copy (rows k,
//            columns gN..gN+N), sB = the forward block scale read transposed
//   wgrad:   A = column-wise dY (rows n), B = column-wise X (rows k), both from column c_g, 128-token
//            blocks restarting at each expert with an fp32 scale per (row, block) on both operands
//
// Main loop: BK = 128 contraction bytes (one promotion slice) per step; global -> registers (prefetch of
// the next step) -> LDS (16-byte chunks XOR-swizzled by row) -> MFMA operands.  Each of the four waves
// owns a 64x64 quarter of the tile as 4x4 16x16 fragments, with an fp32 partial and an fp32 accumulator
// per fragment.
//
// Two operand feeds (same tiling, same LDS staging of the FP8 bytes):
//  * precise (default): each 32-element piece is widened exactly to bf16 and multiplied on
//    v_mfma_f32_16x16x32_bf16, whose sums are fp32-accurate;
//  * full-rate FP8: v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) at twice the rate.  Lane l feeds
//    row l % 16 with 16-byte chunks g and 4 + g of the 128-byte row (g = l / 16).  Measured on gfx950,
//    it truncates the products of each run of 8 consecutive operand bytes toward zero below a 2^-13
//    window of the run's largest product, so its error is bounded by about 7 * 2^-13 times the largest
//    product of each run rather than by fp32 rounding.
#include "common.h"

namespace mxmoe {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kMaxGroups = 1024;

struct TileInfo {
  int g;          // expert
  int mt, nt;     // tile coordinates inside the expert
  int64_t row0;   // first global row of A for this expert (forward / dgrad)
  int rows;       // valid rows of this tile (forward / dgrad)
  int nblk;       // wgrad: number of 128-token contraction blocks
  int64_t col0;   // wgrad: first column of the expert in the column-wise layout
  bool valid;
};

// Tiles are enumerated expert by expert; inside an expert the output-column tile runs fastest so
// that consecutive workgroups share A rows.  Wave 0 computes the per-expert tile counts and their
// prefix sums in LDS, then every thread binary-searches its tile.
__device__ TileInfo decode_tile(int mode, int wblk, const GemmArgs& p, int32_t* pre, int64_t* rowstart) {
  const int G = p.G;
  const int64_t M = p.M;
  const int nt_count = (int)((mode == kFwd ? p.N : p.K) / BN);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t carry = 0;
    for (int g0 = 0; g0 <= G; g0 += 64) {
      int g = g0 + lane;
      int32_t cnt = 0;
      int64_t o0 = 0;
      if (g <= G) {
        o0 = clamp_off(p.offs[g], M);
        rowstart[g] = o0;
      }
      if (g < G) {
        int64_t o1 = clamp_off(p.offs[g + 1], M);
        int64_t m = o1 > o0 ? o1 - o0 : 0;
        if (mode == kWgrad) cnt = (int32_t)((m + wblk - 1) / wblk);   // contraction blocks (prefix -> c_g)
        else cnt = (int32_t)((m + BM - 1) / BM) * nt_count;
      }
      int32_t incl = cnt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int32_t t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
      }
      if (g <= G) pre[g] = carry + incl - cnt;
      carry += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  TileInfo ti;
  ti.valid = false;
  ti.nblk = 0;
  ti.col0 = 0;
  ti.rows = 0;
  ti.row0 = 0;
  const int64_t t = blockIdx.x;
  if (mode == kWgrad) {
    const int per_g = (int)(p.N / BM) * (int)(p.K / BN);
    const int g = (int)(t / per_g);
    if (g >= G) return ti;
    const int lt = (int)(t % per_g);
    const int ntc = (int)(p.K / BN);
    ti.g = g;
    ti.mt = lt / ntc;
    ti.nt = lt % ntc;
    ti.col0 = (int64_t)wblk * pre[g];
    int64_t o0 = rowstart[g], o1 = rowstart[g + 1];
    ti.nblk = o1 > o0 ? (int)((o1 - o0 + wblk - 1) / wblk) : 0;
    ti.row0 = o0;
    ti.rows = (int)(o1 > o0 ? o1 - o0 : 0);   // contraction length m_g
    ti.valid = true;
    return ti;
  }
  if (t >= pre[G]) return ti;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int lt = (int)(t - pre[g]);
  ti.g = g;
  ti.mt = lt / nt_count;
  ti.nt = lt % nt_count;
  ti.row0 = rowstart[g] + (int64_t)ti.mt * BM;
  int64_t left = rowstart[g + 1] - ti.row0;
  ti.rows = (int)(left < BM ? left : BM);
  ti.valid = ti.rows > 0;
  return ti;
}

// LDS byte offset of 16-byte chunk c of tile row r (8 chunks per 128-byte row).
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

// Eight E4M3 bytes -> eight bf16 multiplied by the power of two whose exponent field is that of
// `scale` (1.0 here: the fp32 scales are applied at promotion); exact.
__device__ __forceinline__ v8bf widen8(uint2 w, float scale) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, scale, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, scale, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, scale, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, scale, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int MODE, int FEED>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const TileInfo& ti, uint8_t* ldsA, uint8_t* ldsB,
                                          uint32_t* ldsSA, uint32_t* ldsSB) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- per-tile operand geometry ------------------------------------------------------------
  // A rows: forward/dgrad -> token rows (clamped to the expert's last row); wgrad -> n rows
  // B rows: forward -> gN + j; dgrad -> k rows of W^c (column offset gN); wgrad -> k rows (col c_g)
  int64_t a_col0 = 0, b_col0 = 0;
  constexpr int WBLK = 128;   // wgrad contraction block (128 tokens)
  int64_t L;   // contraction length in bytes (multiple of 128 for forward/dgrad)
  if (MODE == kFwd) L = p.K;
  else if (MODE == kDgrad) L = p.N;
  else L = (int64_t)WBLK * ti.nblk;
  if (MODE == kDgrad) b_col0 = (int64_t)ti.g * p.N;
  int nblk = ti.nblk;
  if (MODE == kWgrad) {
    a_col0 = ti.col0;
    b_col0 = ti.col0;
    // offsets that are not monotone could place an expert past the leading dimension: clip
    const int64_t room = p.lda > a_col0 ? (p.lda - a_col0) / WBLK : 0;
    if (nblk > room) nblk = (int)room;
    L = (int64_t)WBLK * nblk;
  }
  const int nsteps = (int)((L + BK - 1) / BK);

  // global load assignment: chunk id c = tid + 256 j (j = 0..3): row c / 8, chunk c % 8
  const int ld_row = tid >> 3, ld_ch = tid & 7;
  const uint8_t* a_ptr[4];
  const uint8_t* b_ptr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = ld_row + 32 * j;
    int64_t arow;
    if (MODE == kWgrad) arow = (int64_t)ti.mt * BM + r;
    else arow = ti.row0 + (r < ti.rows ? r : ti.rows - 1);
    a_ptr[j] = p.a + arow * p.lda + a_col0 + ld_ch * 16;
    int64_t brow;
    if (MODE == kFwd) brow = (int64_t)ti.g * p.N + (int64_t)ti.nt * BN + r;
    else brow = (int64_t)ti.nt * BN + r;
    b_ptr[j] = p.b + brow * p.ldb + b_col0 + ld_ch * 16;
  }
  // scale rows: threads 0..127 -> A row tid, 128..255 -> B row tid-128
  const bool s_is_a = tid < 128;
  const int s_r = tid & 127;
  int64_t s_row;
  if (s_is_a) {
    if (MODE == kWgrad) s_row = (int64_t)ti.mt * BM + s_r;
    else s_row = ti.row0 + (s_r < ti.rows ? s_r : ti.rows - 1);
  } else {
    if (MODE == kFwd) s_row = (int64_t)ti.g * p.N + (int64_t)ti.nt * BN + s_r;
    else s_row = (int64_t)ti.nt * BN + s_r;
  }
  const int64_t s_ld = s_is_a ? p.ldsa : p.ldsb;
  const int64_t s_col0 = (s_is_a ? a_col0 : b_col0) / 128;

  uint4 ra[4], rb[4];
  uint32_t rs = 0;

  auto load_step = [&](int ks) {
    const int64_t koff = (int64_t)ks * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bool ok = true;
      if (MODE == kWgrad) ok = (koff + ld_ch * 16) < L;     // chunk inside the expert's blocks
      ra[j] = ok ? *(const uint4*)(a_ptr[j] + koff) : make_uint4(0, 0, 0, 0);
      rb[j] = ok ? *(const uint4*)(b_ptr[j] + koff) : make_uint4(0, 0, 0, 0);
    }
    // A row scales; wgrad also B row scales (forward / dgrad read the B block scale per tile)
    const float* sp = (const float*)(s_is_a ? p.sa : p.sb);
    if (s_is_a || MODE == kWgrad) rs = __float_as_uint(sp[s_row * s_ld + s_col0 + ks]);
  };
  auto store_step = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int r = ld_row + 32 * j;
      *(uint4*)(ldsA + lds_off(r, ld_ch)) = ra[j];
      *(uint4*)(ldsB + lds_off(r, ld_ch)) = rb[j];
    }
    if (s_is_a) ldsSA[s_r] = rs;
    else if (MODE == kWgrad) ldsSB[s_r] = rs;
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fg = lane >> 4;
  if (nsteps > 0) load_step(0);
  for (int ks = 0; ks < nsteps; ++ks) {
    store_step();
    __syncthreads();
    if (ks + 1 < nsteps) load_step(ks + 1);

    // blockwise: fp32 weight-block scale of this step (one per 128x128 block)
    float sbw = 1.f;
    float rsc[4][4], csc[4];
    {
      const float* sw = (const float*)p.sb;
      if (MODE == kFwd) sbw = sw[(((int64_t)ti.g * p.N + (int64_t)ti.nt * BN) / 128) * p.ldsb + ks];
      else if (MODE == kDgrad) sbw = sw[(((int64_t)ti.g * p.N) / 128 + ks) * p.ldsb + ti.nt];
      // promotion factors of the lane's four output rows per A fragment (times the weight-block scale)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rsc[i][q] = __uint_as_float(ldsSA[wm * 64 + i * 16 + 4 * fg + q]) * sbw;
      // wgrad: the lane's output column of each B fragment has its own scale (the X row scale)
#pragma unroll
      for (int j = 0; j < 4; ++j) csc[j] = MODE == kWgrad ? __uint_as_float(ldsSB[wn * 64 + j * 16 + fr]) : 1.f;
    }

    if (FEED == kFeedPrecise) {
      // four bf16 MFMAs of K = 32 per step: lane group fg supplies bytes [8 fg, 8 fg + 8) of each
      // 32-element piece, widened exactly to bf16, so every product is exact and the MFMA sums them at
      // fp32 precision into the slice's partial
      v4f part[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        v8bf af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 64 + i * 16 + fr;
          const uint2 w = *(const uint2*)(ldsA + lds_off(r, 2 * kb + (fg >> 1)) + 8 * (fg & 1));
          af[i] = widen8(w, 1.0f);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = wn * 64 + j * 16 + fr;
          const uint2 w = *(const uint2*)(ldsB + lds_off(r, 2 * kb + (fg >> 1)) + 8 * (fg & 1));
          bfr[j] = widen8(w, 1.0f);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], part[i][j], 0, 0, 0);
      }
      // promotion of the slice's partial with its two fp32 scales
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float f = MODE == kWgrad ? rsc[i][q] * csc[j] : rsc[i][q];
            acc[i][j][q] = __builtin_fmaf(part[i][j][q], f, acc[i][j][q]);
          }
    } else {
      // full-rate FP8 MFMA (unit scales), K = 128 per instruction: one unscaled partial per slice
      v8i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + fr;
        v4i lo = *(const v4i*)(ldsA + lds_off(r, fg));
        v4i hi = *(const v4i*)(ldsA + lds_off(r, 4 + fg));
        af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wn * 64 + i * 16 + fr;
        v4i lo = *(const v4i*)(ldsB + lds_off(r, fg));
        v4i hi = *(const v4i*)(ldsB + lds_off(r, 4 + fg));
        bf[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      // promotion: unscaled partial over this 128-slice, then fp32 FMA with the two scales
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], v4f{0.f, 0.f, 0.f, 0.f},
                                                                            0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float f = MODE == kWgrad ? rsc[i][q] * csc[j] : rsc[i][q];
            acc[i][j][q] = __builtin_fmaf(part[q], f, acc[i][j][q]);
          }
        }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*(l/16)+q of each 16x16 sub-tile, column l%16 --------------
  const int64_t nout = (MODE == kFwd) ? p.N : p.K;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm * 64 + i * 16 + 4 * fg + q;
        const int c = wn * 64 + j * 16 + fr;
        int64_t idx;
        if (MODE == kWgrad) {
          idx = ((int64_t)ti.g * p.N + (int64_t)ti.mt * BM + r) * p.K + (int64_t)ti.nt * BN + c;
        } else {
          if (r >= ti.rows) continue;
          idx = (ti.row0 + r) * nout + (int64_t)ti.nt * BN + c;
        }
        const float v = acc[i][j][q];
        if (p.out_bf16) ((uint16_t*)p.out)[idx] = (uint16_t)f32_to_bf16_bits(v);
        else ((float*)p.out)[idx] = v;
      }
}

template <int MODE, int FEED>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ int32_t pre[kMaxGroups + 1];
  __shared__ int64_t rowstart[kMaxGroups + 1];
  __shared__ __attribute__((aligned(16))) uint8_t ldsA[BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t ldsB[BN * BK];
  __shared__ uint32_t ldsSA[BM];
  __shared__ uint32_t ldsSB[BN];
  const TileInfo ti = decode_tile(MODE, 128, p, pre, rowstart);
  if (!ti.valid) return;   // uniform across the workgroup
  gemm_tile<MODE, FEED>(p, ti, ldsA, ldsB, ldsSA, ldsSB);
}

static int64_t tile_upper_bound(int mode, const GemmArgs& p) {
  if (mode == kWgrad) return (int64_t)p.G * (p.N / BM) * (p.K / BN);
  const int64_t ntc = (mode == kFwd ? p.N : p.K) / BN;
  return ((p.M + BM - 1) / BM + p.G) * ntc;   // sum_g ceil(m_g/BM) <= ceil(M/BM) + G
}

template <int MODE>
static void launch_feed(const GemmArgs& p, dim3 grid, dim3 block, hipStream_t st) {
  if (p.feed == kFeedFast) hipLaunchKernelGGL((grouped_gemm_kernel<MODE, kFeedFast>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((grouped_gemm_kernel<MODE, kFeedPrecise>), grid, block, 0, st, p);
}

hipError_t launch_bw_gemm(int mode, const GemmArgs& p, hipStream_t st) {
  const int64_t tiles = tile_upper_bound(mode, p);
  if (tiles == 0) return hipSuccess;
  dim3 grid((unsigned)tiles), block(kThreads);
  if (mode == kFwd) launch_feed<kFwd>(p, grid, block, st);
  else if (mode == kDgrad) launch_feed<kDgrad>(p, grid, block, st);
  else launch_feed<kWgrad>(p, grid, block, st);
  return hipGetLastError();
}

}  // namespace mxmoe
