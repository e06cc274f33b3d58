// MX grouped GEMM of a dropless MoE expert layer on gfx950: forward, dgrad and wgrad in one launch
// each, every expert on its real number of rows (iitak.ru, "NVIDIA sped up training of
// mixture-of-experts models on JAX tenfold": one call for all experts, real token counts, no capacity
// padding, no dropped tokens; opensourcebeat.com MXFP8/DeepEP article, section "Two-sided attack":
// MXFP8 applied to the grouped GEMMs of the expert layers).
//
// Generic form computed by one workgroup, output tile (mt, nt) of expert g:
//   out[i, j] = sum_t A[row_a(i), col0 + t] * B[row_b(j), col0_b + t],   t < L_g
// with a per-32 E8M0 scale on each operand, where
//   forward: A = X rows of expert g, B = W_g rows (gN + n), L = K           (Y = X W^T)
//   dgrad:   A = dY rows of expert g, B = column-wise W (rows k, columns gN..gN+N), L = N
//   wgrad:   A = column-wise dY (rows n), B = column-wise X (rows k), both from column c_g,
//            L = 32 ceil(m_g / 32); the zero pad columns of the layout contribute nothing
//
// Tiling: 256 x 256 output tile per workgroup of 8 waves (2 along A rows x 4 along B rows, 128 x 64
// outputs per wave).  The contraction advances 128 bytes (four MX blocks) per stage.  Operand bytes
// and scale bytes go global -> LDS by direct-to-LDS loads (no register staging), two stages in LDS:
// the loads of stage s+1 are issued early in stage s, after the barrier that publishes it, and land
// while stage s is multiplied (the precise feed issues them after its first 32-block's MFMAs, the FP8
// feed inside its first MFMA group, so that a stage opens with LDS reads).  Each load is a per-tile
// 32-bit lane offset from a wave-uniform base in scalar registers that advances by the stage, so
// issuing costs no vector arithmetic.  LDS rows are 128 bytes with 16-byte chunks XOR-swizzled by
// row.  A column-wise operand may be in the 128-byte tiled layout (a stage of a row is then one
// 128-byte piece of tile ks; the stage advance is the operand's chunk stride).  The output tile leaves
// through LDS as whole row pieces (store_tile_rows).
//
// Operand feeds (same tiling and LDS staging):
//  * precise (default): each lane reads 16 consecutive bytes of one MX block, widens them exactly to
//    bf16 with the block's power-of-two scale folded in (v_cvt_scalef32_pk_bf16_fp8), and feeds two
//    v_mfma_f32_32x32x16_bf16; every product is exact and the MFMA sums at fp32 precision.  A and B
//    use the same assignment of contraction elements to MFMA k-slots, so the sum is unchanged.
//  * fast (opt-in, the *_fp8feed entry points): v_mfma_scale_f32_32x32x64_f8f6f4 at twice the bf16
//    rate, scales applied by the instruction, two k-steps per stage (lane layout at the loop).  Its
//    sums are truncated per run of 8 products (see include/mxmoe.h).
//
// MXFP4 (E2M1 codes two per byte, E8M0 per 32): the same tiling with 128 bytes = 256 elements
// (eight blocks) per stage on the fast feed only, two v_mfma_scale_f32_16x16x128_f8f6f4 k-steps per
// fragment pair and stage with the E2M1 operand format; lane l feeds row l % 16 with the 16 bytes of
// block g (k-step 0) and 4 + g (k-step 1), g = l / 16, and that block's scale (measured on gfx950).
// E2M1 products span at most 2^-2 .. 36 times the pair's scales, inside the instruction's summation
// window, so its sums are exact up to fp32 accumulation.
//
// Scheduling: the tile list of the launch is built on the device from the group offsets (prefix sums
// in LDS); forward / dgrad enumerate ceil(m_g / 256) row tiles per expert, so an expert without rows
// has no tile and a 17-row expert one; wgrad has ceil(N/256) x ceil(K/256) tiles for every expert
// (zeros for an empty one), experts taken largest first.  Inside an expert tiles are rasterised in
// columns of four A tiles; consecutive chunks of 8 tiles go to the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs) so that tiles sharing operands share an L2.
#include "grouped_tile.h"

namespace mxmoe {
namespace {

using Tile = GroupTile;

constexpr int BM = 256;                          // A rows per tile
constexpr int BN = 256;                          // B rows per tile (output columns)
constexpr int BK = 128;                          // contraction elements (bytes) per stage
constexpr int kWavesM = 2;                       // waves along the A rows of the tile
constexpr int kWavesN = 4;                       // waves along the B rows
constexpr int kWaves = kWavesM * kWavesN;
constexpr int NT = 64 * kWaves;                  // threads per workgroup
constexpr int WM = BM / kWavesM;                 // outputs per wave along A rows
constexpr int WN = BN / kWavesN;                 // outputs per wave along B rows
constexpr int kLoadRows = BM / kWaves;           // A (and B) rows each wave loads per stage
constexpr int kScaleLoads = 2 * BM / 64 / kWaves;  // dword scale loads (64 rows each) per wave
constexpr int kScaleRows = 2 * BM / NT;          // scale rows each thread gathers (register path)
static_assert(BM == BN && kLoadRows % 8 == 0 && kScaleLoads >= 1 && kScaleRows >= 1, "tile / wave layout");
constexpr int kStageA = BM * BK;                 // 32 KiB
constexpr int kStage = kStageA + BN * BK;        // 64 KiB
constexpr int kScaleStage = (BM + BN) * 4;       // four E8M0 bytes per operand row (E4M3)
constexpr int kScaleStage4 = (BM + BN) * 8;      // eight E8M0 bytes per operand row (E2M1), two dword planes
constexpr int kLds = 2 * kStage + 2 * kScaleStage4;

typedef float v16f __attribute__((ext_vector_type(16)));


// LDS rows of 128 bytes; 16-byte chunk c of row r sits at chunk position c ^ swz(r), so that the
// lanes of one 16-byte LDS read (consecutive rows, same logical chunk) hit distinct banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 4); }

// Gated forward epilogue (precise feed, 32x32 fragments, 8 waves 2 x 4).  Waves wn = 0, 1 hold the
// gate columns of the tile's 128 hidden units, waves 2, 3 the up columns of the same units.  Every
// wave writes its pre-activations as bf16 to Y (gate at column u, up at H + u).  Then each gate wave
// and the up wave holding the same outputs swap half of their fp32 values through LDS, and each forms
// H = silu(gate) * up in fp32 for its half of the rows and MX-quantises it row-wise: a row's 32-column
// block is one fragment, split between lanes l and l ^ 32.  (Waves w and w + 4, the two row halves of
// one column group, share a SIMD: with the gate waves alone doing this, two SIMDs would sit idle
// through the exponentials.)  With a column-wise output every wave puts its H transposed into LDS, and
// all waves then quantise the tile's 256 rows x 128 hidden units in 32-row blocks down each column (the
// tile's rows start at a multiple of 256 inside its expert, so its blocks are the expert's blocks).
template <typename Acc>
__device__ __forceinline__ void act_epilogue(const GemmArgs& p, const Tile& t, char* lds, Acc (&acc)[WM / 32][WN / 32]) {
  constexpr int NI = WM / 32, NJ = WN / 32;
  constexpr int kUpPitch = BN / 2 + 4;            // floats per LDS row (padded against bank conflicts)
  static_assert(BM * kUpPitch * 4 <= kLds, "exchanged values must fit in LDS");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / kWavesN, wn = w % kWavesN;
  const int64_t H = p.N / 2;
  const bool up_wave = wn >= kWavesN / 2;
  const bool colwise = p.act_qT != nullptr;       // uniform: a kernel argument
  const int ucol0 = WN * (wn % (kWavesN / 2)) + 4 * (lane / 32);    // tile-local hidden column of fragment 0
  const int64_t hcol0 = (int64_t)t.nt * (BN / 2) + ucol0;          // global hidden column
  const int row_lim = t.rows;
  const int lrow = WM * wm + lane % 32;

  // pre-activations (bf16) as whole row pieces through LDS (store_tile_rows): gate waves at columns
  // [128 nt, +128) of Y, up waves at H + the same
  stage_barrier();                                  // every wave is done with the last stage
  static_assert(kWaves * 64 * (128 * NJ + 16) <= kLds, "staged Y must fit in LDS");
  store_tile_rows<NI, NJ, 2>(acc, lds + w * 64 * (128 * NJ + 16), true, p.out, t.row0, p.N,
                             (up_wave ? H : 0) + (int64_t)t.nt * (BN / 2), WM * wm, WN * (wn % (kWavesN / 2)),
                             row_lim, BN);
  // Exchange through LDS, so that every SIMD forms H for half of its rows (a SIMD holds the two row
  // halves of one column group: both gate waves or both up waves).  Gate waves keep fragment rows
  // i < NI / 2 and hand over their gate values of i >= NI / 2; up waves keep i >= NI / 2 and hand over
  // their up values of i < NI / 2.  Both go to xch[r][c] (tile row r, tile-local hidden column c):
  // the two halves are disjoint.  The region is free once every wave is done with its staged rows.
  constexpr int kHalf = NI / 2;
  float* xch = (float*)lds;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if ((i < kHalf) != up_wave) continue;          // a fragment row this wave keeps
    const int r = lrow + 32 * i;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = ucol0 + 32 * j + 8 * q;
        *(float4*)(xch + r * kUpPitch + c) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // H = silu(gate) * up for the kept rows, MX-quantised row-wise; H replaces the kept accumulators
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if ((i < kHalf) == up_wave) continue;          // a fragment row handed over
    const int r = lrow + 32 * i;
    const int64_t grow = t.row0 + r;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float h[16];
      uint32_t amax = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 o = *(const float4*)(xch + r * kUpPitch + ucol0 + 32 * j + 8 * q);
        const float oo[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float mine = acc[i][j][4 * q + k];
          const float g = up_wave ? oo[k] : mine, u = up_wave ? mine : oo[k];
          // silu with the hardware exponential and reciprocal (a few ulp; g -> -inf gives -0)
          h[4 * q + k] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          amax = max(amax, __float_as_uint(h[4 * q + k]) & 0x7FFFFFFFu);
          acc[i][j][4 * q + k] = h[4 * q + k];
        }
      }
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
      // shared exponent of the block: floor(log2 amax) - 8 from the fp32 exponent field, clamped
      const int e = max((int)(amax >> 23) - 135, -127);
      const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
      const float lim = __uint_as_float(((uint32_t)(e + 135) << 23) | 0x600000u);   // 448 * 2^e
      if (r >= row_lim) continue;
      const int64_t hc = hcol0 + 32 * j;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t code = cvt4_f32_e4m3_scaled(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3], lim, sc);
        *(uint32_t*)(p.act_q + grow * H + hc + 8 * q) = code;
        if (p.act_dbg)
          *(float4*)(p.act_dbg + grow * H + hc + 8 * q) = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
      }
      if (lane < 32) {
        // row-wise scales [M, H / 32], or tiled [H / 128][M][4]
        const int64_t blk = (hc - 4 * (lane / 32)) / 32;
        const int64_t off = p.act_tiled ? (blk >> 2) * (p.M * 4) + grow * 4 + (blk & 3) : grow * (H / 32) + blk;
        p.act_s[off] = (uint8_t)(e + 127);
      }
    }
  }
  if (!colwise) return;

  // Column-wise H.  H goes to LDS transposed, column c of the tile at hT + c * kTPitch with its 256
  // rows contiguous (every exchanged value has been read: one more barrier first).  Then 16 lanes take one
  // hidden column: at step m lane k reads the column's 16-byte chunk 16 m + k (rows 4 (16 m + k) .. + 3),
  // so 32-row block b = 2 m + k / 8 is held by 8 lanes, whose amax meets by DPP, and the 16 lanes store
  // 64 consecutive code bytes of the column's qT row.  Blocks at or past the expert's end within this
  // tile hold no rows of it (the next expert's columns) and are skipped; rows past its end inside its
  // last block are pads (zero codes).
  constexpr int kTPitch = BM + 8;                 // the two lane halves of a transposed store: disjoint banks
  static_assert((BN / 2) * kTPitch * 4 <= kLds, "transposed H must fit in LDS");
  float* hT = (float*)lds;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if ((i < kHalf) == up_wave) continue;          // H of the rows this wave kept
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) hT[(ucol0 + 32 * j + 8 * q + k) * kTPitch + lrow + 32 * i] = acc[i][j][4 * q + k];
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const int64_t ldq = p.act_ld;
  // byte of qT row u, column j: row-major [H, ldq], or tiled [ldq / 128][H][128]
  auto qt_at = [&](int64_t u, int64_t j) -> int64_t {
    return p.act_tiled ? (j >> 7) * (H * 128) + u * 128 + (j & 127) : u * ldq + j;
  };
  // scale byte of qT row u, block b: row-major [H, ldq / 32], or tiled [ldq / 128][H][4]
  auto st_at = [&](int64_t u, int64_t b) -> int64_t {
    return p.act_tiled ? (b >> 2) * (H * 4) + u * 4 + (b & 3) : u * (ldq / 32) + b;
  };
  const int64_t tcol = t.col0 + (int64_t)t.mt * BM;               // the tile's first column of qT
  const int nb_tile = (row_lim + 31) / 32;
  const int k16 = lane & 15;
  for (int cb = 4 * w + (lane >> 4); cb < BN / 2; cb += 4 * kWaves) {
    const int64_t u = (int64_t)t.nt * (BN / 2) + cb;              // hidden unit: row of qT
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row0 = 4 * (16 * m + k16);
      const float4 x = *(const float4*)(hT + cb * kTPitch + row0);
      const float v0 = row0 < row_lim ? x.x : 0.f, v1 = row0 + 1 < row_lim ? x.y : 0.f;
      const float v2 = row0 + 2 < row_lim ? x.z : 0.f, v3 = row0 + 3 < row_lim ? x.w : 0.f;
      uint32_t amax = max(max(__float_as_uint(v0) & 0x7FFFFFFFu, __float_as_uint(v1) & 0x7FFFFFFFu),
                          max(__float_as_uint(v2) & 0x7FFFFFFFu, __float_as_uint(v3) & 0x7FFFFFFFu));
      amax = oct_max(amax);
      const int e = max((int)(amax >> 23) - 135, -127);
      const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
      const float lim = __uint_as_float(((uint32_t)(e + 135) << 23) | 0x600000u);
      const uint32_t code = cvt4_f32_e4m3_scaled(v0, v1, v2, v3, lim, sc);
      const int b = 2 * m + (k16 >> 3);
      // (with offsets that are not monotone an expert's blocks could lie past the leading dimension)
      if (b < nb_tile && tcol + 32 * b + 32 <= ldq) {
        *(uint32_t*)(p.act_qT + qt_at(u, tcol + row0)) = code;
        if ((k16 & 7) == 0) p.act_sT[st_at(u, tcol / 32 + b)] = (uint8_t)(e + 127);
      }
    }
  }
  // the tile holding the last routed row zeroes the tail of its 128 rows of qT and sT: the columns past
  // the last expert's blocks
  if (t.row0 + t.rows == p.M) {
    const int64_t tail = ldq - t.col_end;                           // a multiple of 32
    const int64_t chunks = tail / 16;
    for (int64_t k = tid; k < (BN / 2) * chunks; k += NT) {
      const int64_t u = (int64_t)t.nt * (BN / 2) + k / chunks;
      *(uint4*)(p.act_qT + qt_at(u, t.col_end + 16 * (k % chunks))) = make_uint4(0, 0, 0, 0);
    }
    const int64_t stail = tail / 32;
    for (int64_t k = tid; k < (BN / 2) * stail; k += NT) {
      const int64_t u = (int64_t)t.nt * (BN / 2) + k / stail;
      p.act_sT[st_at(u, t.col_end / 32 + k % stail)] = 0;
    }
  }
}

// BWP2: blockwise operands with power-of-two fp32 scales (the SDW path): one fp32 per row and
// 128-element stage for A (1x128 tiles) and for both wgrad operands (128-token blocks), per 128x128
// block for the forward / dgrad B.  Such a scale is exactly the E8M0 scale 2^(exponent field - 127),
// so its exponent byte, repeated for the stage's four 32-blocks, takes the place of the MX scale word
// and the stage multiplies exactly as an MX stage.  The wgrad tile list counts 128-token blocks
// (experts start on a 128-column boundary of the blockwise layout).
template <int MODE, int FEED, bool SDW, bool FP4, bool ACT, bool BWP2 = false>
__device__ __forceinline__ void run_tile(const GemmArgs& p, const Tile& t, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  static_assert(!FP4 || FEED == kFeedFast, "E2M1 operands use the block-scaled MFMA");
  // E2M1: two elements per byte, so a 128-byte stage holds eight 32-blocks
  constexpr int EPB = FP4 ? 2 : 1;            // elements per byte
  constexpr int SPS = FP4 ? 8 : 4;            // scale bytes per row and stage
  // Weight gradient with direct-to-LDS scale loads (scale rows of aligned dwords): an expert's blocks
  // start at an arbitrary block of the column-wise layout.  Its contraction starts f = (first block)
  // mod 4 blocks earlier, at a block whose scale byte opens an aligned dword (the same f for every row
  // of the tile: all belong to one expert), so every stage's scale bytes are whole dwords.  The f
  // leading blocks of the first stage are not loaded: their operand chunks are zeroed and their scale
  // bytes masked to 0, so they add exact zeros.
  constexpr bool ALIGNED_START = MODE == kWgrad && SDW;
  static_assert(!(ALIGNED_START && FP4), "the E2M1 weight gradient gathers its scale rows in registers");
  constexpr int kSStage = FP4 ? kScaleStage4 : kScaleStage;

  // ---- operand geometry (contraction offsets in bytes; scale offsets in 32-blocks) ------------
  const int f = ALIGNED_START && t.nblk > 0 ? (int)((t.col0 / 32) & 3) : 0;   // leading blocks
  // wgrad: 32-blocks looped over (BWP2: the tile list counts 128-token blocks, and f == 0)
  const int nblk_e = (BWP2 ? 4 : 1) * t.nblk + f;
  int64_t L;
  if (MODE == kFwd) L = p.K / EPB;
  else if (MODE == kDgrad) L = p.N / EPB;
  else L = 32 / EPB * (int64_t)nblk_e;
  const int nsteps = (int)((L + BK - 1) / BK);
  const int64_t L0 = 32 / EPB * f;                        // bytes of the leading blocks (first stage)
  const int64_t a_el0 = MODE == kWgrad ? t.col0 - 32 * f : 0;     // first contraction element
  const int64_t b_el0 = MODE == kWgrad ? t.col0 - 32 * f : (MODE == kDgrad ? (int64_t)t.g * p.N : 0);
  const int64_t a_col0 = a_el0 / EPB, b_col0 = b_el0 / EPB;
  const int64_t a_rows_lim = MODE == kWgrad ? p.N : 0;     // wgrad: A rows are n
  const int64_t b_rows_lim = MODE == kFwd ? p.N : p.K;

  auto a_row = [&](int r) -> int64_t {
    if (MODE == kWgrad) return min((int64_t)t.mt * BM + r, a_rows_lim - 1);
    return t.row0 + min(r, t.rows - 1);
  };
  auto b_row = [&](int r) -> int64_t {
    if (ACT) {
      // gated forward: tile columns [0, 128) are gate rows 128 nt .., [128, 256) the up rows of the
      // same hidden units (N = 2H, up rows start at H)
      const int64_t n = (r < BN / 2 ? 0 : p.N / 2 - BN / 2) + (int64_t)t.nt * (BN / 2) + r;
      return (int64_t)t.g * p.N + n;
    }
    const int64_t n = min((int64_t)t.nt * BN + r, b_rows_lim - 1);
    return MODE == kFwd ? (int64_t)t.g * p.N + n : n;
  };

  // data loads: wave w moves rows [R w, R w + R) of A and of B (R = kLoadRows), 8 rows (1 KiB) per
  // instruction; lane l lands in row R w + 8j + l/8 at chunk position l%8, which holds logical chunk
  // (l%8) ^ swz(row)
  constexpr int ND = kLoadRows / 8;
  const int drow = kLoadRows * w + (lane >> 3);
  auto dchunk = [&](int j) { return (lane & 7) ^ swz(drow + 8 * j); };
  // operand rows of the tile relative to its first row (rows never decrease with r): a uniform base per
  // operand and a 32-bit byte offset per lane and load (the host keeps the span of 256 rows, or of the
  // gated forward's N weight rows, below 2 GiB)
  // (contraction byte k of a row sits at chunk k / 128, byte k % 128: chunks are a_kstride / b_kstride
  // bytes apart, 128 in the row-major layouts; the tiled column-wise layout starts every expert's
  // contraction, and so a_col0 / b_col0, at a multiple of 128)
  const uint8_t* a_base = p.a + a_row(0) * p.lda + (a_col0 >> 7) * p.a_kstride + (a_col0 & 127);
  const uint8_t* b_base = p.b + b_row(0) * p.ldb + (b_col0 >> 7) * p.b_kstride + (b_col0 & 127);
  uint32_t a_off[ND], b_off[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    a_off[j] = (uint32_t)((a_row(drow + 8 * j) - a_row(0)) * p.lda) + 16 * dchunk(j);
    b_off[j] = (uint32_t)((b_row(drow + 8 * j) - b_row(0)) * p.ldb) + 16 * dchunk(j);
  }
  // scale loads: four E8M0 bytes per row and stage, landing as one dword per row (A rows then B
  // rows).  When the four bytes are an aligned dword in memory (forward, dgrad), the 512 rows move
  // as 8 direct-to-LDS dword loads of 64 rows (u < 4: A rows [64u, 64u + 64), else B rows), spread
  // over the waves; the weight gradient does the same when its scale rows are aligned
  // (ALIGNED_START above).  Otherwise (wgrad: experts start at arbitrary 32-blocks) thread t gathers rows
  // q = t + NT j (q < 256: A row q, else B row q - 256) into registers one stage ahead and stores
  // the dwords to LDS.
  // A row's scale bytes sit in groups of four (one 128-element chunk), sa_gstride / sb_gstride bytes
  // apart: 4 in the row-major layouts (a plain row), rows * 4 in the tiled column-wise layout, where a
  // chunk's groups of all rows form one block ([ld / 128][rows][4]; only with aligned dwords).
  const uint8_t* sa = (const uint8_t*)p.sa;
  const uint8_t* sb = (const uint8_t*)p.sb;
  const int64_t sa_col0 = a_el0 / 32, sb_col0 = b_el0 / 32;
  constexpr int NS = SDW ? kScaleLoads : kScaleRows;
  const uint8_t* s_src[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    int q;
    if (SDW) q = 64 * (kScaleLoads * w + j) + lane;
    else q = tid + NT * j;
    const int r = q & 255;
    s_src[j] = q < 256 ? sa + a_row(r) * p.ldsa + (sa_col0 >> 2) * p.sa_gstride + (sa_col0 & 3)
                       : sb + b_row(r) * p.ldsb + (sb_col0 >> 2) * p.sb_gstride + (sb_col0 & 3);
    if (BWP2 && MODE != kWgrad && q >= 256) {
      // fp32 block scales [G N / 128, K / 128]: row stride ldsb = K / 32 bytes.  Forward: block row
      // (g N + n) / 128, one fp32 per stage.  Dgrad (B rows k, the stages run over n): block column
      // k / 128, block row g N / 128 + stage.
      if (MODE == kFwd) s_src[j] = sb + (b_row(r) >> 7) * p.ldsb;
      else s_src[j] = sb + (((int64_t)t.g * p.N) >> 7) * p.ldsb + (b_row(r) >> 7) * 4;
    }
  }
  // bytes between a row's scale groups (direct-to-LDS paths: 64 rows of one operand per load) and
  // between the scales of consecutive stages (BWP2 dgrad B: one block row of scales)
  int64_t s_gs[NS], s_step[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bool b_rows = (SDW ? 64 * (kScaleLoads * w + j) : tid + NT * j) >= 256;
    s_gs[j] = b_rows ? p.sb_gstride : p.sa_gstride;
    s_step[j] = BWP2 && MODE == kDgrad && b_rows ? p.ldsb : (SPS / 4) * s_gs[j];
  }
  // Scale bytes [SPS ks, SPS ks + nv) of a row (nv < SPS only in the last wgrad stage; the rest read
  // as 0) land as SPS / 4 dwords, dword d of every row in plane d of the stage's scale area.  Register
  // path: aligned dword loads funnel-shifted together; word k is read only when it holds a wanted
  // byte (else the previous word is read again), so no load touches a word without a byte of the
  // row.  The words are combined only when stored, one stage later, so that no wait for them sits
  // between the loads of a stage.
  constexpr int P = SPS / 4;                  // dword planes
  auto scale_geom = [&](int j, int ks, int& nv, int& sh) -> const uint32_t* {
    nv = MODE == kWgrad ? min(SPS, nblk_e - SPS * ks) : SPS;
    const uintptr_t ai = (uintptr_t)(s_src[j] + SPS * ks);
    sh = (int)(ai & 3);
    return (const uint32_t*)(ai & ~(uintptr_t)3);
  };
  auto gather_scales = [&](int ks, uint32_t (*sw)[P + 1]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      int nv, sh;
      typedef const __attribute__((address_space(1))) uint32_t* gptr;
      const gptr w0 = (gptr)scale_geom(j, ks, nv, sh);
      sw[j][0] = w0[0];
#pragma unroll
      for (int k = 1; k <= P; ++k) sw[j][k] = w0[4 * k < sh + nv ? k : k - 1];
    }
  };
  auto put_scales = [&](int ks, const uint32_t (*sw)[P + 1]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      int nv, sh;
      scale_geom(j, ks, nv, sh);
#pragma unroll
      for (int d = 0; d < P; ++d) {
        uint32_t v = __builtin_amdgcn_alignbyte(sw[j][d + 1], sw[j][d], (uint32_t)sh);
        const int keep = nv - 4 * d;            // valid bytes of this dword
        if (keep <= 0) v = 0;
        else if (keep < 4) v &= (1u << (8 * keep)) - 1u;
        *(uint32_t*)(lds + 2 * kStage + (ks & 1) * kSStage + 2048 * d + 4 * (tid + NT * j)) = v;
      }
    }
  };

  // Loads of stage ks into buffer ks % 2 (which no wave reads any more): issue_rows moves chunk row j of
  // both operands (the FP8 loop issues them inside its first MFMA group), issue_scales the stage's
  // scale bytes.
  auto issue_rows = [&](int ks, int j) {
    char* st = lds + (ks & 1) * kStage;
    // wgrad: chunks outside the expert's blocks, bytes [lim_lo, lim_hi) of the stage's rows, are not
    // loaded (zeroed where they would have landed)
    const int64_t koff = (int64_t)ks * BK;
    const int lim_hi = (int)min(L - koff, (int64_t)BK);
    const int lim_lo = ks == 0 ? (int)L0 : 0;
    const int c = 16 * dchunk(j);
    if (MODE != kWgrad || (c < lim_hi && c >= lim_lo)) {
      dma16s(a_off[j], a_base + (int64_t)ks * p.a_kstride, st + (kLoadRows * w + 8 * j) * BK);
      dma16s(b_off[j], b_base + (int64_t)ks * p.b_kstride, st + kStageA + (kLoadRows * w + 8 * j) * BK);
    } else {
      // a chunk outside the expert's blocks: zeros where the load would have landed (the buffer is
      // free when a stage is issued, and the barrier that publishes the stage waits for LDS stores)
      *(uint4*)(st + (kLoadRows * w + 8 * j) * BK + 16 * lane) = make_uint4(0, 0, 0, 0);
      *(uint4*)(st + kStageA + (kLoadRows * w + 8 * j) * BK + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
  };
  auto issue_scales = [&](int ks) {
    char* ss = lds + 2 * kStage + (ks & 1) * kSStage;
    if constexpr (ALIGNED_START) {
      // the stage's first scale dword, and the second (E2M1) only when the stage's blocks reach into
      // it (so no load passes the expert's bytes of the row)
      const int nv = min(SPS, nblk_e - SPS * ks);
#pragma unroll
      for (int d = 0; d < SPS / 4; ++d) {
        if (d == 0 || nv > 4 * d) {
#pragma unroll
          for (int j = 0; j < NS; ++j)
            dma4(s_src[j] + ((SPS / 4) * ks + d) * s_gs[j], ss + 2048 * d + 256 * (kScaleLoads * w + j));
        }
      }
    } else if (SDW) {
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int d = 0; d < P; ++d)
          dma4(s_src[j] + s_step[j] * ks + d * s_gs[j], ss + 2048 * d + 256 * (kScaleLoads * w + j));
    }
  };

  // ---- accumulators ----------------------------------------------------------------------------
  const int wm = w / kWavesN, wn = w % kWavesN;
  // A wave whose 128 A rows all lie past the tile's valid rows (the last row tile of an expert with at
  // most 128 rows left; the last N tile of a weight gradient with N % 256 == 128) skips its LDS reads
  // and MFMAs: it still moves its share of every stage's loads and meets every barrier, and the other
  // wave of its column, on the same SIMD, has the matrix core to itself.  Its accumulators stay zero
  // and its rows are not stored.
  const int valid_rows = MODE == kWgrad ? (int)min((int64_t)BM, p.N - (int64_t)t.mt * BM) : t.rows;
  const bool active = __builtin_amdgcn_readfirstlane((int)(WM * wm < valid_rows)) != 0;
  constexpr int FR = FP4 ? 16 : 32;                       // fragment rows / columns (E2M1: 16x16x128)
  constexpr int NI = WM / FR;                            // A fragments
  constexpr int NJ = WN / FR;                            // B fragments
  constexpr int NR = FR * FR / 64;                       // accumulator registers per fragment pair
  typedef float vacc __attribute__((ext_vector_type(NR)));
  vacc acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.f;

  uint32_t s_w[NS][P + 1];                       // register-staged scale words of the next stage
  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < ND; ++j) issue_rows(0, j);
    issue_scales(0);
    if (!SDW) {
      gather_scales(0, s_w);
      put_scales(0, s_w);
      if (nsteps > 1) gather_scales(1, s_w);
    }
  }
  // The stage's blocks [lo_b, hi_b) belong to the expert: the leading blocks (first stage) and those past
  // its last block (last stage) were not loaded (their chunks were zeroed at issue).  With ALIGNED_START
  // the scale bytes of the other blocks are masked to 0 (a stale 0xFF would read as NaN): keep[] holds
  // the wave-uniform byte masks of the stage's scale words.
  auto stage_keep = [&](int ks, uint32_t (&keep)[SPS / 4]) {
    const int lo_b = ks == 0 ? f : 0;
    const int hi_b = MODE == kWgrad ? min(SPS, nblk_e - SPS * ks) : SPS;
#pragma unroll
    for (int d = 0; d < SPS / 4; ++d) {
      auto low = [](int k) { return k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u); };
      keep[d] = __builtin_amdgcn_readfirstlane(low(hi_b - 4 * d) & ~low(lo_b - 4 * d));
    }
  };
  auto sword_k = [&](const uint32_t* S, int r, const uint32_t (&keep)[SPS / 4], int word = 0) -> uint32_t {
    if constexpr (BWP2) {
      return ((S[r] >> 23) & 0xFFu) * 0x01010101u;      // the power of two's exponent byte, 4 blocks
    } else if constexpr (ALIGNED_START) {
      return S[512 * word + r] & keep[word];
    } else {
      return S[512 * word + r];
    }
  };
  // Loads of stage s into buffer s % 2, which no wave reads any more.  Register-staged scale words: those
  // of stage s arrived earlier; they are stored, and stage s + 1's gathered, before the operand loads go
  // out (a wait the compiler places for those registers counts only its own loads, while the hardware
  // counter would also hold the operand loads issued after them).
  auto stage_out = [&](int s, bool rows) {
    if (!SDW) put_scales(s, s_w);
    if (!SDW && s + 1 < nsteps) gather_scales(s + 1, s_w);
    if (rows) {
#pragma unroll
      for (int j = 0; j < ND; ++j) issue_rows(s, j);
    }
    issue_scales(s);
  };

  for (int ks = 0; ks < nsteps; ++ks) {
    stage_barrier();                               // stage ks landed; stage ks-1 fully read
    // The next stage's loads may go out any time after the barrier (its buffer was last read in stage
    // ks - 1) and must land by the next barrier.  The precise feed issues them after its first block's
    // MFMAs, so that a stage opens with LDS reads, widening and MFMAs rather than with the issue.  The
    // FP8 feed issues its scale loads at the top and its operand loads inside its first MFMA group,
    // after that group's LDS reads: a stage then opens with LDS reads rather than with eight loads
    // (fast-feed GEMMs of the expert shard 3-6% faster for forward and dgrad, wgrad within 1%).
    // Measured and dropped: spreading the precise feed's loads over its blocks, one chunk row per
    // group of MFMAs or two per block (4-9% slower; a probe of the bare loop had shown 4% more MFMA
    // issue per clock), and a software-pipelined precise loop, with the next block's LDS reads issued
    // before the current block's MFMAs and the stage barrier moved before the last block's MFMAs
    // (4-7% slower).
    const bool more = ks + 1 < nsteps;
    // An idle wave (see `active`) only issues its share of the next stage.  The FP8 and E2M1 feeds
    // issue from one place (a second copy of the register-staged scale path measured a third slower on
    // the E2M1 weight gradient); the precise feed keeps its issue after the first block.
    constexpr bool kFastTop = FP4;
    if constexpr (FEED != kFeedPrecise) {
      if (more) stage_out(ks + 1, kFastTop || !active);
      if (!active) continue;
    } else if (!active) {
      // (a test of `active` at each of the precise feed's four blocks instead measured 1% slower)
      if (more) stage_out(ks + 1, true);
      continue;
    }
    const char* A = lds + (ks & 1) * kStage;
    const char* B = A + kStageA;
    const uint32_t* SA = (const uint32_t*)(lds + 2 * kStage + (ks & 1) * kSStage);
    const uint32_t* SB = SA + BM;
    uint32_t keep[SPS / 4];
    stage_keep(ks, keep);
    auto sword = [&](const uint32_t* S, int r, int word = 0) -> uint32_t { return sword_k(S, r, keep, word); };
    if constexpr (FEED == kFeedPrecise) {
      const int lr = lane & 31, h = lane >> 5;
      uint32_t sa_w[NI], sb_w[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i) sa_w[i] = sword(SA, WM * wm + 32 * i + lr);
#pragma unroll
      for (int j = 0; j < NJ; ++j) sb_w[j] = sword(SB, WN * wn + 32 * j + lr);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        v8bf alo[NI], ahi[NI], blo[NJ], bhi[NJ];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r = WM * wm + 32 * i + lr;
          const uint4 v = *(const uint4*)(A + lds_off(r, 2 * bb + h));
          const float sc = e8m0_as_scale(sa_w[i], bb);
          alo[i] = widen8(v.x, v.y, sc);
          ahi[i] = widen8(v.z, v.w, sc);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int r = WN * wn + 32 * j + lr;
          const uint4 v = *(const uint4*)(B + lds_off(r, 2 * bb + h));
          const float sc = e8m0_as_scale(sb_w[j], bb);
          blo[j] = widen8(v.x, v.y, sc);
          bhi[j] = widen8(v.z, v.w, sc);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(blo[j], alo[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bhi[j], ahi[i], acc[i][j], 0, 0, 0);
        if (more && bb == 0) stage_out(ks + 1, true);
      }
    } else if constexpr (FP4) {
      // two k-steps of 128 E2M1 elements: lane group fg feeds block 4 ks2 + fg (16 bytes, the upper
      // half of the operand registers unused) with its scale byte from plane ks2
      const int fr = lane & 15, fg = lane >> 4;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        v8i bf[NJ];
        int sbv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int r = WN * wn + 16 * j + fr;
          const v4i c = *(const v4i*)(B + lds_off(r, 4 * ks2 + fg));
          bf[j] = v8i{c[0], c[1], c[2], c[3], 0, 0, 0, 0};
          sbv[j] = (int)((sword(SB, r, ks2) >> (8 * fg)) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r = WM * wm + 16 * i + fr;
          const v4i c = *(const v4i*)(A + lds_off(r, 4 * ks2 + fg));
          const v8i af = v8i{c[0], c[1], c[2], c[3], 0, 0, 0, 0};
          const int sav = (int)((sword(SA, r, ks2) >> (8 * fg)) & 0xFFu);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 4, 4, 0, sbv[j], 0, sav);
        }
      }
    } else {
      // E4M3 on v_mfma_scale_f32_32x32x64_f8f6f4, two k-steps of 64 bytes per stage.  Lane l feeds row
      // l % 32 with the 16-byte chunks 4 ks2 + h and 4 ks2 + 2 + h of the 128-byte row (h = l / 32); the
      // scale operand of half h applies to the stage's block 2 ks2 + h, i.e. to chunks 4 ks2 + 2h and
      // 4 ks2 + 2h + 1, which lanes of both halves hold (measured on gfx950).
      const int lr = lane & 31, h = lane >> 5;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        v8i bf[NJ];
        int sbv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int r = WN * wn + 32 * j + lr;
          const v4i lo = *(const v4i*)(B + lds_off(r, 4 * ks2 + h));
          const v4i hi = *(const v4i*)(B + lds_off(r, 4 * ks2 + 2 + h));
          bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          sbv[j] = (int)((sword(SB, r) >> (8 * (2 * ks2 + h))) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r = WM * wm + 32 * i + lr;
          const v4i lo = *(const v4i*)(A + lds_off(r, 4 * ks2 + h));
          const v4i hi = *(const v4i*)(A + lds_off(r, 4 * ks2 + 2 + h));
          const v8i af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const int sav = (int)((sword(SA, r) >> (8 * (2 * ks2 + h))) & 0xFFu);
          if (!kFastTop && more && ks2 == 0 && i == 0) {
#pragma unroll
            for (int q = 0; q < ND; ++q) issue_rows(ks + 1, q);
          }
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0, sbv[j], 0, sav);
        }
      }
    }
  }

  if constexpr (ACT) {
    static_assert(MODE == kFwd && FEED == kFeedPrecise && !FP4, "gated epilogue: precise forward only");
    act_epilogue(p, t, lds, acc);
    return;
  }

  // ---- epilogue --------------------------------------------------------------------------------
  // The MFMAs take the B fragment as their first operand, so each accumulator holds a tile transposed:
  // lane l has output row (fragment row) l % 32 (l % 16 for the 16x16 shape) and, per group of four
  // registers, four consecutive output columns, written with one 8-byte (bf16) or 16-byte (fp32)
  // store.  Output row of tile row rl: forward / dgrad row0 + rl of [M, nout]; wgrad n = mt*BM + rl
  // of dW_g [N, K].  N and K are multiples of 128, so no group of four columns straddles the edge.
  const int64_t nout = MODE == kFwd ? p.N : p.K;
  const int row_lim = (int)min((int64_t)BM, MODE == kWgrad ? p.N - (int64_t)t.mt * BM : (int64_t)t.rows);
  const int col_lim = (int)min((int64_t)BN, nout - (int64_t)t.nt * BN);
  const int64_t out_row0 = MODE == kWgrad ? (int64_t)t.g * p.N + (int64_t)t.mt * BM : t.row0;
  constexpr int FI = FR;                                 // fragment rows / columns
  const int lrow = WM * wm + lane % FI;
  const int lcol = WN * wn + 4 * (lane / FI);
  const int64_t base = (out_row0 + lrow) * nout + (int64_t)t.nt * BN + lcol;
  if constexpr (FR == 32 && NI % 2 == 0) {
    // E4M3 (32x32 fragments): through LDS, 64 rows of each wave at a time (store_tile_rows; measured:
    // the expert-shard step -1.4%, the DeepSeek-V3-16B step -3% against stores straight from the
    // accumulators).  Every wave is done with the stages once it has passed the barrier.
    static_assert(kWaves * 64 * (128 * NJ + 16) <= kLds, "staged epilogue must fit in LDS");
    stage_barrier();
    store_tile_rows<NI, NJ, 2>(acc, lds + w * 64 * (128 * NJ + 16), p.out_bf16, p.out, out_row0, nout,
                               (int64_t)t.nt * BN, WM * wm, WN * wn, row_lim, col_lim);
    return;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (lrow + FI * i >= row_lim) continue;
    const int64_t rbase = base + (int64_t)(FI * i) * nout;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        const int co = FI * j + 8 * q;                     // 32x32: register group q covers columns 8q + 4h .. + 3
        if (lcol + co >= col_lim) continue;
        const int64_t idx = rbase + co;
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (p.out_bf16) {
          const uint2 w = make_uint2(f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16),
                                     f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16));
          *(uint2*)((uint16_t*)p.out + idx) = w;
        } else {
          *(float4*)((float*)p.out + idx) = make_float4(v0, v1, v2, v3);
        }
      }
  }
}

template <int MODE, int FEED, bool SDW, bool FP4 = false, bool ACT = false, bool BWP2 = false>
__global__ __launch_bounds__(NT, 1) void mx_grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  Tile t;
  // (the blockwise power-of-two wgrad lays experts out in 128-token blocks)
  if (!decode_grouped_tile<MODE, MODE == kWgrad || ACT, BM, BN, NT, BWP2 ? 128 : 32, MODE != kWgrad>(p, lds, t))
    return;
  // the tile's fields are the same in every lane: say so, so that everything derived from them (operand
  // bases, loop bounds) lives in scalar registers
  t.g = __builtin_amdgcn_readfirstlane(t.g);
  t.mt = __builtin_amdgcn_readfirstlane(t.mt);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);
  t.nblk = __builtin_amdgcn_readfirstlane(t.nblk);
  t.row0 = uniform64(t.row0);
  t.col0 = uniform64(t.col0);
  t.col_end = uniform64(t.col_end);
  __syncthreads();                               // scheduler scratch is reused for operands
  run_tile<MODE, FEED, SDW, FP4, ACT, BWP2>(p, t, lds);
}

static_assert(5 * (kMaxG + 1) * 4 <= kStage, "scheduler scratch must fit in the first stage");

int64_t tile_count_bound(int mode, const GemmArgs& p) {
  if (mode == kWgrad) return (int64_t)p.G * ((p.N + BM - 1) / BM) * ((p.K + BN - 1) / BN);
  const int64_t ntc = ((mode == kFwd ? p.N : p.K) + BN - 1) / BN;
  return ((p.M + BM - 1) / BM + p.G) * ntc;     // sum_g ceil(m_g / BM) <= ceil(M / BM) + G
}

template <int MODE, bool SDW>
void launch_mode(const GemmArgs& p, dim3 grid, hipStream_t st) {
  if (p.fp4)
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<MODE, kFeedFast, SDW, true>), grid, dim3(NT), 0, st, p);
  else if (p.feed == kFeedFast)
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<MODE, kFeedFast, SDW>), grid, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<MODE, kFeedPrecise, SDW>), grid, dim3(NT), 0, st, p);
}

}  // namespace

hipError_t launch_mx_gemm(int mode, const GemmArgs& args, hipStream_t st) {
  GemmArgs p = args;
  if (p.a_kstride == 0) p.a_kstride = BK;        // row-major operands
  if (p.b_kstride == 0) p.b_kstride = BK;
  if (p.sa_gstride == 0) p.sa_gstride = 4;       // row-major scale rows
  if (p.sb_gstride == 0) p.sb_gstride = 4;
  // tiled scale layouts are read only by the direct-to-LDS dword paths (E4M3, scale rows of dwords)
  const bool tiled_scales = p.sa_gstride != 4 || p.sb_gstride != 4;
  if (tiled_scales && (p.fp4 || p.bw_pow2 || p.ldsa % 4 || p.ldsb % 4)) return hipErrorInvalidValue;
  const int64_t tiles = tile_count_bound(mode, p);
  if (tiles == 0) return hipSuccess;
  const int64_t per = (int64_t)kXcd * chunk_tiles(mode);   // whole XCD chunks: every tile has a workgroup
  const int64_t grid = (tiles + per - 1) / per * per;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  // the scale bytes of a row and stage are aligned dwords when every scale row and column offset is
  // a multiple of 4 bytes (wgrad expert columns start at arbitrary 32-blocks)
  p.scale_dword = mode != kWgrad && p.ldsa % 4 == 0 && p.ldsb % 4 == 0 && (p.N / 32) % 4 == 0;
  if (tiled_scales && mode != kWgrad && !p.scale_dword) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid);
  if (p.bw_pow2) {
    // blockwise operands with power-of-two scales: scale rows of aligned dwords
    if (p.fp4 || p.act_q || p.ldsa % 4 || p.ldsb % 4 || (mode != kWgrad && !p.scale_dword)) return hipErrorInvalidValue;
    if (mode == kWgrad && p.feed == kFeedFast)
      hipLaunchKernelGGL((mx_grouped_gemm_kernel<kWgrad, kFeedFast, true, false, false, true>), g, dim3(NT), 0, st, p);
    else if (mode == kWgrad)
      hipLaunchKernelGGL((mx_grouped_gemm_kernel<kWgrad, kFeedPrecise, true, false, false, true>), g, dim3(NT), 0, st, p);
    else if (mode == kFwd && p.feed == kFeedFast)
      hipLaunchKernelGGL((mx_grouped_gemm_kernel<kFwd, kFeedFast, true, false, false, true>), g, dim3(NT), 0, st, p);
    else if (mode == kFwd)
      hipLaunchKernelGGL((mx_grouped_gemm_kernel<kFwd, kFeedPrecise, true, false, false, true>), g, dim3(NT), 0, st, p);
    else if (p.feed == kFeedFast)
      hipLaunchKernelGGL((mx_grouped_gemm_kernel<kDgrad, kFeedFast, true, false, false, true>), g, dim3(NT), 0, st, p);
    else
      hipLaunchKernelGGL((mx_grouped_gemm_kernel<kDgrad, kFeedPrecise, true, false, false, true>), g, dim3(NT), 0, st, p);
    return hipGetLastError();
  }
  if (mode == kFwd && p.act_q) {
    if (!p.scale_dword) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<kFwd, kFeedPrecise, true, false, true>), g, dim3(NT), 0, st, p);
  } else if (mode == kFwd) launch_mode<kFwd, true>(p, g, st);
  else if (mode == kDgrad && p.scale_dword) launch_mode<kDgrad, true>(p, g, st);
  else if (mode == kDgrad) launch_mode<kDgrad, false>(p, g, st);
  else if (!p.fp4 && p.ldsa % 4 == 0 && p.ldsb % 4 == 0 && p.feed == kFeedPrecise)
    // E4M3 scale rows of aligned dwords (a row pitch that is a multiple of 128): direct-to-LDS scale
    // loads from an aligned-down start
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<kWgrad, kFeedPrecise, true>), g, dim3(NT), 0, st, p);
  else if (!p.fp4 && p.ldsa % 4 == 0 && p.ldsb % 4 == 0)
    hipLaunchKernelGGL((mx_grouped_gemm_kernel<kWgrad, kFeedFast, true>), g, dim3(NT), 0, st, p);
  else launch_mode<kWgrad, false>(p, g, st);
  return hipGetLastError();
}

}  // namespace mxmoe
