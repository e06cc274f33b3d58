// Blockwise-FP8 dropless grouped GEMM for MoE experts on gfx950 (the DeepSeek-V3 fine-grained recipe).
//
// aifind.ru, "DeepSeek-V3: a revolutionary high-performance language model with low training cost", section
// "Low-precision training: FP8 Framework", captions (a) and (b): activations carry an fp32 scale per 1x128
// tile, weights per 128x128 block, and the FP8 products are summed over each 128-element slice of the
// contraction before that partial is promoted, i.e. multiplied by its two scales and added to a
// full-precision accumulator.  All experts run in one launch, each on its real number of rows (iitak.ru,
// "NVIDIA sped up training of mixture-of-experts models on JAX tenfold": no capacity padding, no dropped
// tokens).
//
// Generic form computed by one workgroup (tile (mt, nt) of expert g), promoted per 128-slice kb:
//   out[i, j] = sum_kb sA(i, kb) sB(j, kb) sum_{t in kb} A[row_a(i), col0_a + t] * B[row_b(j), col0_b + t]
// where
//   forward: A = X rows of expert g, B = W_g rows; sA = the 1x128 tile scale, sB = the 128x128 block scale
//            (one per tile and slice: a tile's 128 B rows are one weight block row)
//   dgrad:   A = dY rows of expert g (1x128 tiles along N), B = the transposed weight copy (rows k,
//            columns gN..gN+N); sB = the forward block scale of (n-slice kb, k-block nt)
//   wgrad:   A = column-wise dY (rows n), B = column-wise X (rows k), both from column c_g, 128-token
//            blocks restarting at each expert; sA, sB the row scales of each block (sB per output column)
//
// The MX kernel's design with a 256 x 128 tile: 8 waves of 64 x 64 outputs (4 along A rows x 2 along B
// rows), so each wave keeps an fp32 partial beside its accumulators (64 + 64 registers).  A stage is one
// promotion slice (128 contraction bytes); operand rows and fp32 row scales move global -> LDS by
// direct-to-LDS loads from a wave-uniform base and per-tile 32-bit lane offsets, two stages in LDS with
// one barrier per stage, the next stage's loads issued after the first 32 elements' MFMAs.  LDS rows
// of 128 bytes with 16-byte chunks XOR-swizzled by row.  The tile list comes from the device-resident
// offsets (grouped_tile.h): ceil(m_g / 256) x (N_out / 128) tiles per expert for forward / dgrad (none
// for an empty expert), every (n, k) tile of every expert for wgrad, largest expert first.
//
// Operand feeds:
//  * precise (default): each lane widens 16 E4M3 bytes exactly to bf16 and feeds two
//    v_mfma_f32_32x32x16_bf16 per 32 elements, whose sums are fp32-accurate;
//  * full-rate FP8: v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales, two k-steps per slice (lane
//    l: row l % 32, chunks 4 s + h and 4 s + 2 + h, h = l / 32).  Measured on gfx950, it truncates the
//    products of each run of 8 consecutive operand bytes toward zero to a 2^-13 window of the run's
//    largest product, so its error is bounded by about 7 * 2^-13 times the largest product of each run.
#include "grouped_tile.h"

namespace mxmoe {
namespace {

constexpr int BM = 256;                          // A rows per tile
constexpr int BN = 128;                          // B rows per tile (output columns)
constexpr int BK = 128;                          // contraction bytes per stage: one promotion slice
constexpr int kWavesM = 4, kWavesN = 2, kWaves = kWavesM * kWavesN;
constexpr int NT = 64 * kWaves;
constexpr int WM = BM / kWavesM, WN = BN / kWavesN;          // 64 x 64 outputs per wave
constexpr int NI = WM / 32, NJ = WN / 32;                    // 32 x 32 fragments
constexpr int kRowsA = BM / kWaves, kRowsB = BN / kWaves;    // operand rows each wave loads per stage
constexpr int NDA = kRowsA / 8, NDB = kRowsB / 8;            // 1 KiB loads (8 rows) per wave and stage
constexpr int kStageA = BM * BK;                             // 32 KiB
constexpr int kStage = kStageA + BN * BK;                    // 48 KiB
constexpr int kScaleA = 0, kScaleB = 4 * BM, kScaleBlk = 4 * (BM + BN);   // byte offsets in a scale stage
constexpr int kScaleStage = 4 * (BM + BN) + 16;
constexpr int kLds = 2 * kStage + 2 * kScaleStage;
static_assert(5 * (kMaxG + 1) * 4 <= kStage, "scheduler scratch must fit in the first stage");

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 4); }

template <int MODE, int FEED>
__device__ __forceinline__ void bw_tile(const GemmArgs& p, const GroupTile& t, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w / kWavesN, wn = w % kWavesN;
  const int lr = lane & 31, h = lane >> 5;

  // ---- geometry (contraction offsets in bytes) ------------------------------------------------
  int64_t L;
  if (MODE == kFwd) L = p.K;
  else if (MODE == kDgrad) L = p.N;
  else L = (int64_t)BK * t.nblk;                 // whole 128-token blocks (pad columns hold zero codes)
  const int nsteps = (int)(L / BK);
  const int64_t a_col0 = MODE == kWgrad ? t.col0 : 0;
  const int64_t b_col0 = MODE == kWgrad ? t.col0 : (MODE == kDgrad ? (int64_t)t.g * p.N : 0);
  auto a_row = [&](int r) -> int64_t {
    if (MODE == kWgrad) return min((int64_t)t.mt * BM + r, p.N - 1);
    return t.row0 + min(r, t.rows - 1);
  };
  auto b_row = [&](int r) -> int64_t {
    const int64_t n = min((int64_t)t.nt * BN + r, (MODE == kFwd ? p.N : p.K) - 1);
    return MODE == kFwd ? (int64_t)t.g * p.N + n : n;
  };

  // operand loads: wave w moves A rows [kRowsA w, +kRowsA) and B rows [kRowsB w, +kRowsB), 8 rows per
  // instruction; lane l lands in row (base + l / 8) at chunk position l % 8, which holds logical chunk
  // (l % 8) ^ swz(row)
  const int drow_a = kRowsA * w + (lane >> 3), drow_b = kRowsB * w + (lane >> 3);
  const uint8_t* a_base = p.a + a_row(0) * p.lda + a_col0;
  const uint8_t* b_base = p.b + b_row(0) * p.ldb + b_col0;
  uint32_t a_off[NDA], b_off[NDB];
#pragma unroll
  for (int j = 0; j < NDA; ++j)
    a_off[j] = (uint32_t)((a_row(drow_a + 8 * j) - a_row(0)) * p.lda) + 16 * ((lane & 7) ^ swz(drow_a + 8 * j));
#pragma unroll
  for (int j = 0; j < NDB; ++j)
    b_off[j] = (uint32_t)((b_row(drow_b + 8 * j) - b_row(0)) * p.ldb) + 16 * ((lane & 7) ^ swz(drow_b + 8 * j));
  // fp32 scales, one dword per stage: waves 0-3 load the A row scales of rows [64 w, 64 w + 64); for wgrad
  // waves 4-5 the B row scales of rows [64 (w - 4), +64); for forward / dgrad lane 0 of wave 4 the tile's
  // block scale.  Each lands at its row's dword of the stage's scale area.
  const float* sa = (const float*)p.sa;
  const float* sb = (const float*)p.sb;
  const float* s_src = nullptr;
  int s_dst = -1;
  if (w < 4) {
    s_src = sa + a_row(64 * w + lane) * p.ldsa + a_col0 / BK;
    s_dst = kScaleA + 256 * w;
  } else if (MODE == kWgrad && w < 6) {
    s_src = sb + b_row(64 * (w - 4) + lane) * p.ldsb + b_col0 / BK;
    s_dst = kScaleB + 256 * (w - 4);
  } else if (MODE != kWgrad && w == 4) {
    // forward: block (gN + 128 nt) / 128 of the weight rows, slice ks; dgrad: block row gN / 128 + ks
    // (the n-slice), column nt (the tile's k block)
    if (MODE == kFwd) s_src = sb + (((int64_t)t.g * p.N) / BN + t.nt) * p.ldsb;
    else s_src = sb + (((int64_t)t.g * p.N) / BK) * p.ldsb + t.nt;
    s_dst = kScaleBlk;
  }
  const int64_t s_step = MODE == kDgrad && w == 4 ? p.ldsb : 1;   // floats between the stages' scales

  auto issue = [&](int ks) {
    char* st = lds + (ks & 1) * kStage;
    char* ss = lds + 2 * kStage + (ks & 1) * kScaleStage;
    const int64_t koff = (int64_t)ks * BK;
#pragma unroll
    for (int j = 0; j < NDA; ++j) dma16s(a_off[j], a_base + koff, st + (kRowsA * w + 8 * j) * BK);
#pragma unroll
    for (int j = 0; j < NDB; ++j) dma16s(b_off[j], b_base + koff, st + kStageA + (kRowsB * w + 8 * j) * BK);
    if (s_dst >= 0) {
      if (MODE == kWgrad || w < 4) dma4((const uint8_t*)(s_src + ks), ss + s_dst);
      else if (lane == 0) dma4((const uint8_t*)(s_src + ks * s_step), ss + s_dst);
    }
  };

  // ---- accumulators and the promoted partials -----------------------------------------------
  v16f acc[NI][NJ], part[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nsteps > 0) issue(0);
  for (int ks = 0; ks < nsteps; ++ks) {
    stage_barrier();                               // stage ks landed; stage ks-1 fully read
    constexpr bool kLateIssue = FEED == kFeedPrecise;
    if (!kLateIssue && ks + 1 < nsteps) issue(ks + 1);
    const char* A = lds + (ks & 1) * kStage;
    const char* B = A + kStageA;
    const v16f zero = {};                          // the slice's first MFMAs start from 0 (no zeroing pass)
    if constexpr (FEED == kFeedPrecise) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        v8bf alo[NI], ahi[NI], blo[NJ], bhi[NJ];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const uint4 v = *(const uint4*)(A + lds_off(WM * wm + 32 * i + lr, 2 * bb + h));
          alo[i] = widen8(v.x, v.y, 1.0f);
          ahi[i] = widen8(v.z, v.w, 1.0f);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint4 v = *(const uint4*)(B + lds_off(WN * wn + 32 * j + lr, 2 * bb + h));
          blo[j] = widen8(v.x, v.y, 1.0f);
          bhi[j] = widen8(v.z, v.w, 1.0f);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(blo[j], alo[i], bb == 0 ? zero : part[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bhi[j], ahi[i], part[i][j], 0, 0, 0);
        if (kLateIssue && bb == 0 && ks + 1 < nsteps) issue(ks + 1);
      }
    } else {
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        v8i bf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int r = WN * wn + 32 * j + lr;
          const v4i lo = *(const v4i*)(B + lds_off(r, 4 * ks2 + h));
          const v4i hi = *(const v4i*)(B + lds_off(r, 4 * ks2 + 2 + h));
          bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r = WM * wm + 32 * i + lr;
          const v4i lo = *(const v4i*)(A + lds_off(r, 4 * ks2 + h));
          const v4i hi = *(const v4i*)(A + lds_off(r, 4 * ks2 + 2 + h));
          const v8i af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af, ks2 == 0 ? zero : part[i][j], 0, 0,
                                                                          0, 127, 0, 127);
        }
      }
    }
    // promotion.  The MFMAs take the B fragment first, so lane l holds output row (A row) l % 32 of each
    // fragment, and per group of four registers four consecutive output columns 8q + 4h .. + 3.
    const char* S = lds + 2 * kStage + (ks & 1) * kScaleStage;
    float fa[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) fa[i] = *(const float*)(S + kScaleA + 4 * (WM * wm + 32 * i + lr));
    if constexpr (MODE == kWgrad) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 cb = *(const float4*)(S + kScaleB + 4 * (WN * wn + 32 * j + 8 * q + 4 * h));
          const float cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              acc[i][j][4 * q + k] = __builtin_fmaf(part[i][j][4 * q + k], fa[i] * cbv[k], acc[i][j][4 * q + k]);
        }
    } else {
      const float fb = *(const float*)(S + kScaleBlk);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float fi = fa[i] * fb;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(part[i][j][r], fi, acc[i][j][r]);
      }
    }
  }

  // ---- epilogue: through LDS, 32 rows of each wave at a time, whole row pieces (store_tile_rows) ----
  const int64_t nout = MODE == kFwd ? p.N : p.K;
  const int row_lim = (int)min((int64_t)BM, MODE == kWgrad ? p.N - (int64_t)t.mt * BM : (int64_t)t.rows);
  const int col_lim = (int)min((int64_t)BN, nout - (int64_t)t.nt * BN);
  const int64_t out_row0 = MODE == kWgrad ? (int64_t)t.g * p.N + (int64_t)t.mt * BM : t.row0;
  static_assert(kWaves * 32 * (128 * NJ + 16) <= kLds, "staged epilogue must fit in LDS");
  stage_barrier();                                 // every wave is done with the stages
  store_tile_rows<NI, NJ, 1>(acc, lds + w * 32 * (128 * NJ + 16), p.out_bf16, p.out, out_row0, nout,
                             (int64_t)t.nt * BN, WM * wm, WN * wn, row_lim, col_lim);
}

template <int MODE, int FEED>
__global__ __launch_bounds__(NT, 1) void bw_grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  GroupTile t;
  if (!decode_grouped_tile<MODE, MODE == kWgrad, BM, BN, NT, BK>(p, lds, t)) return;   // uniform
  t.g = __builtin_amdgcn_readfirstlane(t.g);
  t.mt = __builtin_amdgcn_readfirstlane(t.mt);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);
  t.nblk = __builtin_amdgcn_readfirstlane(t.nblk);
  t.row0 = uniform64(t.row0);
  t.col0 = uniform64(t.col0);
  __syncthreads();                               // scheduler scratch is reused for operands
  bw_tile<MODE, FEED>(p, t, lds);
}

int64_t bw_tile_count_bound(int mode, const GemmArgs& p) {
  if (mode == kWgrad) return (int64_t)p.G * ((p.N + BM - 1) / BM) * ((p.K + BN - 1) / BN);
  const int64_t ntc = ((mode == kFwd ? p.N : p.K) + BN - 1) / BN;
  return ((p.M + BM - 1) / BM + p.G) * ntc;     // sum_g ceil(m_g / BM) <= ceil(M / BM) + G
}

template <int MODE>
void bw_launch_mode(const GemmArgs& p, dim3 grid, hipStream_t st) {
  if (p.feed == kFeedFast) hipLaunchKernelGGL((bw_grouped_gemm_kernel<MODE, kFeedFast>), grid, dim3(NT), 0, st, p);
  else hipLaunchKernelGGL((bw_grouped_gemm_kernel<MODE, kFeedPrecise>), grid, dim3(NT), 0, st, p);
}

}  // namespace

hipError_t launch_bw_gemm(int mode, const GemmArgs& p, hipStream_t st) {
  const int64_t tiles = bw_tile_count_bound(mode, p);
  if (tiles == 0) return hipSuccess;
  const int64_t per = (int64_t)kXcd * chunk_tiles(mode);   // whole XCD chunks: every tile has a workgroup
  const int64_t grid = (tiles + per - 1) / per * per;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid);
  if (mode == kFwd) bw_launch_mode<kFwd>(p, g, st);
  else if (mode == kDgrad) bw_launch_mode<kDgrad>(p, g, st);
  else bw_launch_mode<kWgrad>(p, g, st);
  return hipGetLastError();
}

}  // namespace mxmoe
