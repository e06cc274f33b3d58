// C ABI of the MXFP8 expert-GEMM library: host-side argument validation (before any HIP call),
// device check, dispatch to the kernels.  See include/mxmoe.h for the contract of each entry point.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

using namespace mxmoe;

namespace {

thread_local char g_err[512] = "";

mxmoe_status fail(mxmoe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

mxmoe_status ok() {
  g_err[0] = '\0';
  return MXMOE_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// gfx950 check, cached per device ordinal (0 = unknown, 1 = gfx950, 2 = other)
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;

mxmoe_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MXMOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev_ok.size() > dev && g_dev_ok[dev] != 0)
      return g_dev_ok[dev] == 1 ? MXMOE_OK : fail(MXMOE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(MXMOE_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
  const bool is950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev_ok.size() <= dev) g_dev_ok.resize(dev + 1, 0);
    g_dev_ok[dev] = is950 ? 1 : 2;
  }
  return is950 ? MXMOE_OK : fail(MXMOE_ERR_UNSUPPORTED, "device %d (%s) is not gfx950", dev, prop.gcnArchName);
}

mxmoe_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXMOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int32_t kMaxG = 1024;

mxmoe_status check_gemm_common(const char* fn, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                               const void* out, int dt) {
  if (G < 1 || G > kMaxG) return fail(MXMOE_ERR_SHAPE, "%s: G = %d outside [1, %d]", fn, (int)G, (int)kMaxG);
  if (M < 0 || N <= 0 || K <= 0) return fail(MXMOE_ERR_SHAPE, "%s: bad sizes M=%lld N=%lld K=%lld", fn,
                                             (long long)M, (long long)N, (long long)K);
  if (N % 128 || K % 128) return fail(MXMOE_ERR_SHAPE, "%s: N and K must be multiples of 128 (N=%lld K=%lld)", fn,
                                      (long long)N, (long long)K);
  if (M > INT32_MAX) return fail(MXMOE_ERR_SHAPE, "%s: M too large", fn);
  if (dt != MXMOE_F32 && dt != MXMOE_BF16) return fail(MXMOE_ERR_DTYPE, "%s: unknown output dtype %d", fn, dt);
  if (!offs) return fail(MXMOE_ERR_NULL, "%s: offs is NULL", fn);
  if (!out) return fail(MXMOE_ERR_NULL, "%s: output is NULL", fn);
  if (!aligned(offs, 4)) return fail(MXMOE_ERR_ALIGN, "%s: offs not 4-byte aligned", fn);
  if (!aligned(out, 16)) return fail(MXMOE_ERR_ALIGN, "%s: output not 16-byte aligned", fn);
  return MXMOE_OK;
}

mxmoe_status check_ptr(const char* fn, const char* name, const void* p, uintptr_t al) {
  if (!p) return fail(MXMOE_ERR_NULL, "%s: %s is NULL", fn, name);
  if (!aligned(p, al)) return fail(MXMOE_ERR_ALIGN, "%s: %s not %d-byte aligned", fn, name, (int)al);
  return MXMOE_OK;
}

#define TRY(x)                          \
  do {                                  \
    mxmoe_status _s = (x);              \
    if (_s != MXMOE_OK) return _s;      \
  } while (0)

}  // namespace

extern "C" {

int mxmoe_abi_version(void) { return MXMOE_ABI_VERSION; }

const char* mxmoe_last_error(void) { return g_err; }

int64_t mx_colwise_ld_min(int64_t M, int32_t G) {
  if (M < 0 || G < 1) return -1;
  return 32 * ((M + 31 * (int64_t)G + 31) / 32);
}

// A pitch 2^p + 2^(p-k) with k in {7, 8, 9}: p is the position of the highest set bit, and the rest is
// one bit k places below it.
static bool slow_pitch(int64_t ld) {
  if (ld <= 0) return false;
  int p = 63 - __builtin_clzll((unsigned long long)ld);
  const int64_t rest = ld - ((int64_t)1 << p);
  for (int k = 7; k <= 9; ++k)
    if (p >= k && rest == ((int64_t)1 << (p - k))) return true;
  return false;
}

int64_t mxmoe_pitch(int64_t min_ld) {
  if (min_ld < 0) return -1;
  if (min_ld > INT64_MAX - 2048) return min_ld;
  int64_t ld = (min_ld + 127) / 128 * 128;      // scale rows of ld / 32 bytes are then aligned dwords
  while (slow_pitch(ld) && ld <= INT64_MAX - 1024) ld += 1024;
  return ld;
}

static mxmoe_status rowwise_impl(const char* fn, const void* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s,
                                 bool tiled, void* stream) {
  if (R < 0 || C <= 0 || C % 32) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 32 == 0 (R=%lld C=%lld)",
                                            fn, (long long)R, (long long)C);
  if (tiled && C % 128)
    return fail(MXMOE_ERR_SHAPE, "%s: the tiled scale layout needs C %% 128 == 0 (C=%lld)", fn, (long long)C);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "q", q, 16));
  TRY(check_ptr(fn, "s", s, 4));
  TRY(check_device());
  return launched(launch_mx_rowwise((const uint16_t*)x, R, C, q, s, tiled, (hipStream_t)stream), fn);
}

mxmoe_status mx_quantize_rowwise(const void* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, void* stream) {
  return rowwise_impl("mx_quantize_rowwise", x, R, C, q, s, false, stream);
}

mxmoe_status mx_quantize_rowwise_tiled(const void* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, void* stream) {
  return rowwise_impl("mx_quantize_rowwise_tiled", x, R, C, q, s, true, stream);
}

static mxmoe_status colwise_impl(const char* fn, const void* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                                 uint8_t* qT, uint8_t* sT, int64_t ld, bool tiled, void* stream) {
  if (R < 0 || C <= 0 || C % 32) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 32 == 0 (R=%lld C=%lld)",
                                            fn, (long long)R, (long long)C);
  if (R > INT32_MAX) return fail(MXMOE_ERR_SHAPE, "%s: R too large", fn);
  if (offs && (G < 1 || G > kMaxG)) return fail(MXMOE_ERR_SHAPE, "%s: G = %d outside [1, %d]", fn, (int)G, (int)kMaxG);
  if (ld <= 0 || ld % 32) return fail(MXMOE_ERR_ALIGN, "%s: ld must be a positive multiple of 32 (ld=%lld)", fn,
                                      (long long)ld);
  if (tiled && ld % 128)
    return fail(MXMOE_ERR_ALIGN, "%s: the tiled layout needs ld %% 128 == 0 (ld=%lld)", fn, (long long)ld);
  const int64_t need = offs ? mx_colwise_ld_min(R, G) : 32 * ((R + 31) / 32);
  if (ld < need) return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld < required %lld", fn, (long long)ld, (long long)need);
  if (R > 0) TRY(check_ptr(fn, "x", x, 16));
  if (offs && !aligned(offs, 4)) return fail(MXMOE_ERR_ALIGN, "%s: offs not 4-byte aligned", fn);
  TRY(check_ptr(fn, "qT", qT, 16));
  TRY(check_ptr(fn, "sT", sT, 4));
  TRY(check_device());
  return launched(launch_mx_colwise((const uint16_t*)x, R, C, offs, G, qT, sT, ld, tiled, (hipStream_t)stream), fn);
}

mxmoe_status mx_quantize_colwise(const void* x, int64_t R, int64_t C, const int32_t* offs, int32_t G, uint8_t* qT,
                                 uint8_t* sT, int64_t ld, void* stream) {
  return colwise_impl("mx_quantize_colwise", x, R, C, offs, G, qT, sT, ld, false, stream);
}

mxmoe_status mx_quantize_colwise_tiled(const void* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                                       uint8_t* qT, uint8_t* sT, int64_t ld, void* stream) {
  return colwise_impl("mx_quantize_colwise_tiled", x, R, C, offs, G, qT, sT, ld, true, stream);
}

static mxmoe_status dual_impl(const char* fn, const void* x, int64_t R, int64_t C, const int32_t* row_idx,
                              int64_t R_src, const int32_t* offs, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT,
                              uint8_t* sT, int64_t ld, bool tiled, void* stream) {
  if (R < 0 || C <= 0 || C % 32) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 32 == 0 (R=%lld C=%lld)",
                                            fn, (long long)R, (long long)C);
  if (R > INT32_MAX) return fail(MXMOE_ERR_SHAPE, "%s: R too large", fn);
  if (offs && (G < 1 || G > kMaxG)) return fail(MXMOE_ERR_SHAPE, "%s: G = %d outside [1, %d]", fn, (int)G, (int)kMaxG);
  if (ld <= 0 || ld % 32) return fail(MXMOE_ERR_ALIGN, "%s: ld must be a positive multiple of 32 (ld=%lld)", fn,
                                      (long long)ld);
  if (tiled && ld % 128)
    return fail(MXMOE_ERR_ALIGN, "%s: the tiled layout needs ld %% 128 == 0 (ld=%lld)", fn, (long long)ld);
  if (tiled && C % 128)
    return fail(MXMOE_ERR_SHAPE, "%s: the tiled scale layout needs C %% 128 == 0 (C=%lld)", fn, (long long)C);
  const int64_t need = offs ? mx_colwise_ld_min(R, G) : 32 * ((R + 31) / 32);
  if (ld < need) return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld < required %lld", fn, (long long)ld, (long long)need);
  if (row_idx && R > 0 && R_src < 1)
    return fail(MXMOE_ERR_SHAPE, "%s: R_src must be >= 1 with row_idx (R_src=%lld)", fn, (long long)R_src);
  if (R > 0) {
    TRY(check_ptr(fn, "x", x, 16));
    TRY(check_ptr(fn, "q", q, 16));
    TRY(check_ptr(fn, "s", s, 4));
    if (row_idx && !aligned(row_idx, 4)) return fail(MXMOE_ERR_ALIGN, "%s: row_idx not 4-byte aligned", fn);
  }
  if (offs && !aligned(offs, 4)) return fail(MXMOE_ERR_ALIGN, "%s: offs not 4-byte aligned", fn);
  TRY(check_ptr(fn, "qT", qT, 16));
  TRY(check_ptr(fn, "sT", sT, 4));
  TRY(check_device());
  return launched(launch_mx_dual((const uint16_t*)x, R, C, R > 0 ? row_idx : nullptr, row_idx ? R_src : R, offs, G, q,
                                 s, qT, sT, ld, tiled, (hipStream_t)stream),
                  fn);
}

mxmoe_status mx_quantize_dual(const void* x, int64_t R, int64_t C, const int32_t* row_idx, int64_t R_src,
                              const int32_t* offs, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT,
                              int64_t ld, void* stream) {
  return dual_impl("mx_quantize_dual", x, R, C, row_idx, R_src, offs, G, q, s, qT, sT, ld, false, stream);
}

mxmoe_status mx_quantize_dual_tiled(const void* x, int64_t R, int64_t C, const int32_t* row_idx, int64_t R_src,
                                    const int32_t* offs, int32_t G, uint8_t* q, uint8_t* s, uint8_t* qT, uint8_t* sT,
                                    int64_t ld, void* stream) {
  return dual_impl("mx_quantize_dual_tiled", x, R, C, row_idx, R_src, offs, G, q, s, qT, sT, ld, true, stream);
}

// The GEMM addresses a tile's operand rows as 32-bit byte offsets from the tile's first row: 256 rows
// (the gated forward: the N weight rows of an expert) of each operand must span less than 2 GiB, so that
// an offset is the same read as signed or unsigned.
static mxmoe_status check_strides(const char* fn, const GemmArgs& p, int64_t b_rows) {
  const int64_t lim = (int64_t)1 << 31;
  if (256 * p.lda + 256 > lim || b_rows * p.ldb + 256 > lim)
    return fail(MXMOE_ERR_SHAPE, "%s: operand row stride too large (lda=%lld ldb=%lld bytes): a tile's rows must "
                "span less than 2 GiB", fn, (long long)p.lda, (long long)p.ldb);
  return MXMOE_OK;
}

static mxmoe_status mx_gemm_common(int mode, const char* fn, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                   const uint8_t* sb, int64_t ldb_cols, const int32_t* offs, int32_t G, int64_t M,
                                   int64_t N, int64_t K, void* out, int dt, void* stream, int feed,
                                   bool fp4 = false, bool tiled = false) {
  TRY(check_gemm_common(fn, offs, G, M, N, K, out, dt));
  if (fp4 && (N % 256 || K % 256))
    return fail(MXMOE_ERR_SHAPE, "%s: MXFP4 needs N and K multiples of 256 (N=%lld K=%lld)", fn, (long long)N,
                (long long)K);
  TRY(check_ptr(fn, "A operand", a, 16));
  TRY(check_ptr(fn, "A scales", sa, 4));
  TRY(check_ptr(fn, "B operand", b, 16));
  TRY(check_ptr(fn, "B scales", sb, 4));
  GemmArgs p;
  memset(&p, 0, sizeof p);
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.offs = offs; p.out = out;
  p.M = M; p.N = N; p.K = K; p.G = G;
  p.out_bf16 = dt == MXMOE_BF16;
  p.feed = feed;
  // operand leading dimensions in bytes (E2M1: two elements per byte), scale ones in blocks
  const int epb = fp4 ? 2 : 1;
  p.fp4 = fp4;
  if (mode == kFwd) {
    p.lda = K / epb; p.ldsa = K / 32; p.ldb = K / epb; p.ldsb = K / 32;
  } else if (mode == kDgrad) {
    p.lda = N / epb; p.ldsa = N / 32; p.ldb = ldb_cols / epb; p.ldsb = ldb_cols / 32;
  } else {
    p.lda = ldb_cols / epb; p.ldsa = ldb_cols / 32; p.ldb = ldb_cols / epb; p.ldsb = ldb_cols / 32;
  }
  p.a_kstride = p.b_kstride = 128;
  p.sa_gstride = p.sb_gstride = 4;
  if (mode == kWgrad) p.ld_cols = ldb_cols;
  if (tiled) {
    // column-wise operands in the 128-byte tiled layout: rows 128 bytes apart, chunks rows * 128 apart;
    // every scale buffer (row-wise and column-wise) [chunks][rows][4]: rows 4 bytes apart, 4-byte groups
    // rows * 4 apart
    p.ldsa = 4; p.ldsb = 4;
    if (mode == kFwd) {
      p.sa_gstride = 4 * M; p.sb_gstride = 4 * (int64_t)G * N;
    } else if (mode == kDgrad) {
      p.sa_gstride = 4 * M;
      p.ldb = 128; p.b_kstride = 128 * K; p.sb_gstride = 4 * K;
    } else {
      p.lda = 128; p.a_kstride = 128 * N; p.sa_gstride = 4 * N;
      p.ldb = 128; p.b_kstride = 128 * K; p.sb_gstride = 4 * K;
    }
  }
  TRY(check_strides(fn, p, 256));
  if (mode != kWgrad && M == 0) return ok();
  TRY(check_device());
  return launched(launch_mx_gemm(mode, p, (hipStream_t)stream), fn);
}

mxmoe_status mx_grouped_gemm_fwd(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw, const uint8_t* sw,
                                 const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                 mxmoe_dtype ydt, void* stream) {
  return mx_gemm_common(kFwd, "mx_grouped_gemm_fwd", qx, sx, qw, sw, 0, offs, G, M, N, K, y, (int)ydt, stream,
                        kFeedPrecise);
}

mxmoe_status mx_grouped_gemm_fwd_fp8feed(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw, const uint8_t* sw,
                                         const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                         mxmoe_dtype ydt, void* stream) {
  return mx_gemm_common(kFwd, "mx_grouped_gemm_fwd_fp8feed", qx, sx, qw, sw, 0, offs, G, M, N, K, y, (int)ydt,
                        stream, kFeedFast);
}

mxmoe_status mx_grouped_gemm_fwd_tiled(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw, const uint8_t* sw,
                                       const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                       mxmoe_dtype ydt, void* stream) {
  return mx_gemm_common(kFwd, "mx_grouped_gemm_fwd_tiled", qx, sx, qw, sw, 0, offs, G, M, N, K, y, (int)ydt, stream,
                        kFeedPrecise, false, true);
}

mxmoe_status mx_grouped_gemm_fwd_tiled_fp8feed(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw,
                                               const uint8_t* sw, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                               int64_t K, void* y, mxmoe_dtype ydt, void* stream) {
  return mx_gemm_common(kFwd, "mx_grouped_gemm_fwd_tiled_fp8feed", qx, sx, qw, sw, 0, offs, G, M, N, K, y, (int)ydt,
                        stream, kFeedFast, false, true);
}

static mxmoe_status swiglu_impl(const char* fn, const uint8_t* qx, const uint8_t* sx, const uint8_t* qw,
                                const uint8_t* sw, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                void* y, uint8_t* qh, uint8_t* sh, float* h, uint8_t* qhT, uint8_t* shT, int64_t ldh,
                                bool tiled, void* stream) {
  TRY(check_gemm_common(fn, offs, G, M, N, K, y, MXMOE_BF16));
  if (N % 256) return fail(MXMOE_ERR_SHAPE, "%s: N = 2H must be a multiple of 256 (N=%lld)", fn, (long long)N);
  TRY(check_ptr(fn, "A operand", qx, 16));
  TRY(check_ptr(fn, "A scales", sx, 4));
  TRY(check_ptr(fn, "B operand", qw, 16));
  TRY(check_ptr(fn, "B scales", sw, 4));
  TRY(check_ptr(fn, "qh", qh, 16));
  TRY(check_ptr(fn, "sh", sh, 4));
  if (h && !aligned(h, 16)) return fail(MXMOE_ERR_ALIGN, "%s: h not 16-byte aligned", fn);
  if ((qhT == nullptr) != (shT == nullptr)) return fail(MXMOE_ERR_NULL, "%s: qhT and shT go together", fn);
  if (qhT) {
    TRY(check_ptr(fn, "qhT", qhT, 16));
    if (ldh % (tiled ? 128 : 32) || ldh < mx_colwise_ld_min(M, G))
      return fail(MXMOE_ERR_SHAPE, "%s: ldh=%lld must be a multiple of %d and >= mx_colwise_ld_min(M, G)=%lld", fn,
                  (long long)ldh, tiled ? 128 : 32, (long long)mx_colwise_ld_min(M, G));
  } else if (tiled) {
    return fail(MXMOE_ERR_NULL, "%s: the tiled variant writes H column-wise: qhT and shT are required", fn);
  }
  GemmArgs p;
  memset(&p, 0, sizeof p);
  p.a = qx; p.sa = sx; p.b = qw; p.sb = sw; p.offs = offs; p.out = y;
  p.M = M; p.N = N; p.K = K; p.G = G;
  p.out_bf16 = 1;
  p.feed = kFeedPrecise;
  p.lda = K; p.ldsa = K / 32; p.ldb = K; p.ldsb = K / 32;
  p.act_q = qh; p.act_s = sh; p.act_dbg = h;
  p.act_qT = qhT; p.act_sT = shT; p.act_ld = ldh;
  p.act_tiled = tiled;
  p.a_kstride = p.b_kstride = 128;
  p.sa_gstride = p.sb_gstride = 4;
  if (tiled) {
    // row-wise scales of X and W in the tiled layout ([K / 128][M][4], [K / 128][G N][4])
    p.ldsa = 4; p.sa_gstride = 4 * M;
    p.ldsb = 4; p.sb_gstride = 4 * (int64_t)G * N;
  }
  TRY(check_strides(fn, p, N));
  if (M == 0) return ok();
  TRY(check_device());
  return launched(launch_mx_gemm(kFwd, p, (hipStream_t)stream), fn);
}

mxmoe_status mx_grouped_gemm_fwd_swiglu(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw, const uint8_t* sw,
                                        const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                        uint8_t* qh, uint8_t* sh, float* h, uint8_t* qhT, uint8_t* shT, int64_t ldh,
                                        void* stream) {
  return swiglu_impl("mx_grouped_gemm_fwd_swiglu", qx, sx, qw, sw, offs, G, M, N, K, y, qh, sh, h, qhT, shT, ldh,
                     false, stream);
}

mxmoe_status mx_grouped_gemm_fwd_swiglu_tiled(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw,
                                              const uint8_t* sw, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                              int64_t K, void* y, uint8_t* qh, uint8_t* sh, float* h, uint8_t* qhT,
                                              uint8_t* shT, int64_t ldh, void* stream) {
  return swiglu_impl("mx_grouped_gemm_fwd_swiglu_tiled", qx, sx, qw, sw, offs, G, M, N, K, y, qh, sh, h, qhT, shT, ldh,
                     true, stream);
}

static mxmoe_status mx_dgrad_impl(const char* fn, int feed, const uint8_t* qdy, const uint8_t* sdy,
                                  const uint8_t* qwT, const uint8_t* swT, int64_t ldw, const int32_t* offs, int32_t G,
                                  int64_t M, int64_t N, int64_t K, void* dx, mxmoe_dtype dxdt, void* stream,
                                  bool tiled = false) {
  if (ldw % (tiled ? 128 : 32) || ldw < (int64_t)G * N)
    return fail(MXMOE_ERR_SHAPE, "%s: ldw=%lld must be a multiple of %d and >= G*N=%lld", fn, (long long)ldw,
                tiled ? 128 : 32, (long long)G * N);
  return mx_gemm_common(kDgrad, fn, qdy, sdy, qwT, swT, ldw, offs, G, M, N, K, dx, (int)dxdt, stream, feed, false,
                        tiled);
}

mxmoe_status mx_grouped_gemm_dgrad(const uint8_t* qdy, const uint8_t* sdy, const uint8_t* qwT, const uint8_t* swT,
                                   int64_t ldw, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                   void* dx, mxmoe_dtype dxdt, void* stream) {
  return mx_dgrad_impl("mx_grouped_gemm_dgrad", kFeedPrecise, qdy, sdy, qwT, swT, ldw, offs, G, M, N, K, dx, dxdt,
                       stream);
}

mxmoe_status mx_grouped_gemm_dgrad_fp8feed(const uint8_t* qdy, const uint8_t* sdy, const uint8_t* qwT,
                                           const uint8_t* swT, int64_t ldw, const int32_t* offs, int32_t G, int64_t M,
                                           int64_t N, int64_t K, void* dx, mxmoe_dtype dxdt, void* stream) {
  return mx_dgrad_impl("mx_grouped_gemm_dgrad_fp8feed", kFeedFast, qdy, sdy, qwT, swT, ldw, offs, G, M, N, K, dx,
                       dxdt, stream);
}

mxmoe_status mx_grouped_gemm_dgrad_tiled(const uint8_t* qdy, const uint8_t* sdy, const uint8_t* qwT, const uint8_t* swT,
                                         int64_t ldw, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                         void* dx, mxmoe_dtype dxdt, void* stream) {
  return mx_dgrad_impl("mx_grouped_gemm_dgrad_tiled", kFeedPrecise, qdy, sdy, qwT, swT, ldw, offs, G, M, N, K, dx,
                       dxdt, stream, true);
}

mxmoe_status mx_grouped_gemm_dgrad_tiled_fp8feed(const uint8_t* qdy, const uint8_t* sdy, const uint8_t* qwT,
                                                 const uint8_t* swT, int64_t ldw, const int32_t* offs, int32_t G,
                                                 int64_t M, int64_t N, int64_t K, void* dx, mxmoe_dtype dxdt,
                                                 void* stream) {
  return mx_dgrad_impl("mx_grouped_gemm_dgrad_tiled_fp8feed", kFeedFast, qdy, sdy, qwT, swT, ldw, offs, G, M, N, K,
                       dx, dxdt, stream, true);
}

static mxmoe_status mx_wgrad_impl(const char* fn, int feed, const uint8_t* qdyT, const uint8_t* sdyT,
                                  const uint8_t* qxT, const uint8_t* sxT, int64_t ld, const int32_t* offs, int32_t G,
                                  int64_t M, int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt, void* stream,
                                  bool tiled = false) {
  if (G >= 1 && M >= 0 && (ld % (tiled ? 128 : 32) || ld < mx_colwise_ld_min(M, G)))
    return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld must be a multiple of %d and >= mx_colwise_ld_min(M, G)=%lld", fn,
                (long long)ld, tiled ? 128 : 32, (long long)mx_colwise_ld_min(M, G));
  return mx_gemm_common(kWgrad, fn, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw, (int)dwdt, stream, feed, false,
                        tiled);
}

mxmoe_status mx_grouped_gemm_wgrad(const uint8_t* qdyT, const uint8_t* sdyT, const uint8_t* qxT, const uint8_t* sxT,
                                   int64_t ld, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                   void* dw, mxmoe_dtype dwdt, void* stream) {
  return mx_wgrad_impl("mx_grouped_gemm_wgrad", kFeedPrecise, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw, dwdt,
                       stream);
}

mxmoe_status mx_grouped_gemm_wgrad_fp8feed(const uint8_t* qdyT, const uint8_t* sdyT, const uint8_t* qxT,
                                           const uint8_t* sxT, int64_t ld, const int32_t* offs, int32_t G, int64_t M,
                                           int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt, void* stream) {
  return mx_wgrad_impl("mx_grouped_gemm_wgrad_fp8feed", kFeedFast, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw,
                       dwdt, stream);
}

mxmoe_status mx_grouped_gemm_wgrad_tiled(const uint8_t* qdyT, const uint8_t* sdyT, const uint8_t* qxT,
                                         const uint8_t* sxT, int64_t ld, const int32_t* offs, int32_t G, int64_t M,
                                         int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt, void* stream) {
  return mx_wgrad_impl("mx_grouped_gemm_wgrad_tiled", kFeedPrecise, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw,
                       dwdt, stream, true);
}

mxmoe_status mx_grouped_gemm_wgrad_tiled_fp8feed(const uint8_t* qdyT, const uint8_t* sdyT, const uint8_t* qxT,
                                                 const uint8_t* sxT, int64_t ld, const int32_t* offs, int32_t G,
                                                 int64_t M, int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt,
                                                 void* stream) {
  return mx_wgrad_impl("mx_grouped_gemm_wgrad_tiled_fp8feed", kFeedFast, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K,
                       dw, dwdt, stream, true);
}

mxmoe_status mxfp4_quantize_rowwise(const void* x, int64_t R, int64_t C, uint8_t* q, uint8_t* s, void* stream) {
  const char* fn = "mxfp4_quantize_rowwise";
  if (R < 0 || C <= 0 || C % 32) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 32 == 0 (R=%lld C=%lld)",
                                            fn, (long long)R, (long long)C);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "q", q, 16));
  TRY(check_ptr(fn, "s", s, 4));
  TRY(check_device());
  return launched(launch_mxfp4_rowwise((const uint16_t*)x, R, C, q, s, (hipStream_t)stream), fn);
}

mxmoe_status mxfp4_quantize_colwise(const void* x, int64_t R, int64_t C, const int32_t* offs, int32_t G, uint8_t* qT,
                                    uint8_t* sT, int64_t ld, void* stream) {
  const char* fn = "mxfp4_quantize_colwise";
  if (R < 0 || C <= 0 || C % 32) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 32 == 0 (R=%lld C=%lld)",
                                            fn, (long long)R, (long long)C);
  if (R > INT32_MAX) return fail(MXMOE_ERR_SHAPE, "%s: R too large", fn);
  if (offs && (G < 1 || G > kMaxG)) return fail(MXMOE_ERR_SHAPE, "%s: G = %d outside [1, %d]", fn, (int)G, (int)kMaxG);
  if (ld <= 0 || ld % 32) return fail(MXMOE_ERR_ALIGN, "%s: ld must be a positive multiple of 32 (ld=%lld)", fn,
                                      (long long)ld);
  const int64_t need = offs ? mx_colwise_ld_min(R, G) : 32 * ((R + 31) / 32);
  if (ld < need) return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld < required %lld", fn, (long long)ld, (long long)need);
  if (R > 0) TRY(check_ptr(fn, "x", x, 16));
  if (offs && !aligned(offs, 4)) return fail(MXMOE_ERR_ALIGN, "%s: offs not 4-byte aligned", fn);
  TRY(check_ptr(fn, "qT", qT, 16));
  TRY(check_ptr(fn, "sT", sT, 4));
  TRY(check_device());
  return launched(launch_mxfp4_colwise((const uint16_t*)x, R, C, offs, G, qT, sT, ld, (hipStream_t)stream), fn);
}

mxmoe_status mxfp4_grouped_gemm_fwd(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw, const uint8_t* sw,
                                    const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                    mxmoe_dtype ydt, void* stream) {
  return mx_gemm_common(kFwd, "mxfp4_grouped_gemm_fwd", qx, sx, qw, sw, 0, offs, G, M, N, K, y, (int)ydt, stream,
                        kFeedFast, true);
}

mxmoe_status mxfp4_grouped_gemm_dgrad(const uint8_t* qdy, const uint8_t* sdy, const uint8_t* qwT, const uint8_t* swT,
                                      int64_t ldw, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                      void* dx, mxmoe_dtype dxdt, void* stream) {
  const char* fn = "mxfp4_grouped_gemm_dgrad";
  if (ldw % 32 || ldw < (int64_t)G * N)
    return fail(MXMOE_ERR_SHAPE, "%s: ldw=%lld must be a multiple of 32 and >= G*N=%lld", fn, (long long)ldw,
                (long long)G * N);
  return mx_gemm_common(kDgrad, fn, qdy, sdy, qwT, swT, ldw, offs, G, M, N, K, dx, (int)dxdt, stream, kFeedFast,
                        true);
}

mxmoe_status mxfp4_grouped_gemm_wgrad(const uint8_t* qdyT, const uint8_t* sdyT, const uint8_t* qxT,
                                      const uint8_t* sxT, int64_t ld, const int32_t* offs, int32_t G, int64_t M,
                                      int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt, void* stream) {
  const char* fn = "mxfp4_grouped_gemm_wgrad";
  if (G >= 1 && M >= 0 && (ld % 32 || ld < mx_colwise_ld_min(M, G)))
    return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld must be a multiple of 32 and >= mx_colwise_ld_min(M, G)=%lld", fn,
                (long long)ld, (long long)mx_colwise_ld_min(M, G));
  return mx_gemm_common(kWgrad, fn, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw, (int)dwdt, stream, kFeedFast,
                        true);
}

static mxmoe_status bw_act_impl(const char* fn, const void* x, int64_t R, int64_t C, uint8_t* q, float* s, bool pow2,
                                void* stream) {
  if (R < 0 || C <= 0 || C % 128) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 128 == 0", fn);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "q", q, 16));
  TRY(check_ptr(fn, "s", s, 4));
  TRY(check_device());
  return launched(launch_bw_act((const uint16_t*)x, R, C, q, s, pow2, (hipStream_t)stream), fn);
}

mxmoe_status fp8bw_quantize_act_1x128(const void* x, int64_t R, int64_t C, uint8_t* q, float* s, void* stream) {
  return bw_act_impl("fp8bw_quantize_act_1x128", x, R, C, q, s, false, stream);
}

mxmoe_status fp8bw_quantize_act_1x128_pow2(const void* x, int64_t R, int64_t C, uint8_t* q, float* s, void* stream) {
  return bw_act_impl("fp8bw_quantize_act_1x128_pow2", x, R, C, q, s, true, stream);
}

static mxmoe_status bw_weight_impl(const char* fn, const void* w, int64_t R, int64_t C, uint8_t* q, float* s,
                                   uint8_t* qT, bool pow2, void* stream) {
  if (R < 0 || C <= 0 || R % 128 || C % 128)
    return fail(MXMOE_ERR_SHAPE, "%s: need R %% 128 == 0, C > 0, C %% 128 == 0", fn);
  if (R / 128 > 65535 || C / 128 > INT32_MAX) return fail(MXMOE_ERR_SHAPE, "%s: too many blocks", fn);
  if (R == 0) return ok();
  TRY(check_ptr(fn, "w", w, 16));
  TRY(check_ptr(fn, "q", q, 16));
  TRY(check_ptr(fn, "s", s, 4));
  if (qT) TRY(check_ptr(fn, "qT", qT, 16));
  TRY(check_device());
  return launched(launch_bw_weight((const uint16_t*)w, R, C, q, s, qT, pow2, (hipStream_t)stream), fn);
}

mxmoe_status fp8bw_quantize_weight_128x128(const void* w, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT,
                                           void* stream) {
  return bw_weight_impl("fp8bw_quantize_weight_128x128", w, R, C, q, s, qT, false, stream);
}

mxmoe_status fp8bw_quantize_weight_128x128_pow2(const void* w, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT,
                                                void* stream) {
  return bw_weight_impl("fp8bw_quantize_weight_128x128_pow2", w, R, C, q, s, qT, true, stream);
}

int64_t fp8bw_colwise_ld_min(int64_t M, int32_t G) {
  if (M < 0 || G < 1) return -1;
  return 128 * ((M + 127 * (int64_t)G + 127) / 128);
}

static mxmoe_status bw_colwise_impl(const char* fn, const void* x, int64_t R, int64_t C, const int32_t* offs,
                                    int32_t G, uint8_t* qT, float* sT, int64_t ld, bool pow2, void* stream) {
  if (R < 0 || C <= 0 || C % 128) return fail(MXMOE_ERR_SHAPE, "%s: need R >= 0, C > 0, C %% 128 == 0 (R=%lld C=%lld)",
                                             fn, (long long)R, (long long)C);
  if (R > INT32_MAX) return fail(MXMOE_ERR_SHAPE, "%s: R too large", fn);
  if (offs && (G < 1 || G > kMaxG)) return fail(MXMOE_ERR_SHAPE, "%s: G = %d outside [1, %d]", fn, (int)G, (int)kMaxG);
  if (ld <= 0 || ld % 128) return fail(MXMOE_ERR_ALIGN, "%s: ld must be a positive multiple of 128 (ld=%lld)", fn,
                                       (long long)ld);
  const int64_t need = offs ? fp8bw_colwise_ld_min(R, G) : 128 * ((R + 127) / 128);
  if (ld < need) return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld < required %lld", fn, (long long)ld, (long long)need);
  if (R > 0) TRY(check_ptr(fn, "x", x, 16));
  if (offs && !aligned(offs, 4)) return fail(MXMOE_ERR_ALIGN, "%s: offs not 4-byte aligned", fn);
  TRY(check_ptr(fn, "qT", qT, 16));
  TRY(check_ptr(fn, "sT", sT, 4));
  TRY(check_device());
  return launched(launch_bw_colwise((const uint16_t*)x, R, C, offs, G, qT, sT, ld, pow2, (hipStream_t)stream), fn);
}

mxmoe_status fp8bw_quantize_colwise_128(const void* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                                        uint8_t* qT, float* sT, int64_t ld, void* stream) {
  return bw_colwise_impl("fp8bw_quantize_colwise_128", x, R, C, offs, G, qT, sT, ld, false, stream);
}

mxmoe_status fp8bw_quantize_colwise_128_pow2(const void* x, int64_t R, int64_t C, const int32_t* offs, int32_t G,
                                             uint8_t* qT, float* sT, int64_t ld, void* stream) {
  return bw_colwise_impl("fp8bw_quantize_colwise_128_pow2", x, R, C, offs, G, qT, sT, ld, true, stream);
}

static mxmoe_status bw_gemm_common(int mode, const char* fn, int feed, const uint8_t* a, const float* sa,
                                   const uint8_t* b, const float* sb, const int32_t* offs, int32_t G, int64_t M,
                                   int64_t N, int64_t K, void* out, int dt, void* stream, int64_t ld = 0) {
  TRY(check_gemm_common(fn, offs, G, M, N, K, out, dt));
  TRY(check_ptr(fn, "A operand", a, 16));
  TRY(check_ptr(fn, "A scales", sa, 4));
  TRY(check_ptr(fn, "B operand", b, 16));
  TRY(check_ptr(fn, "B scales", sb, 4));
  GemmArgs p;
  memset(&p, 0, sizeof p);
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.offs = offs; p.out = out;
  p.M = M; p.N = N; p.K = K; p.G = G;
  p.out_bf16 = dt == MXMOE_BF16;
  p.feed = feed;
  if (mode == kFwd) {
    p.lda = K; p.ldsa = K / 128; p.ldb = K; p.ldsb = K / 128;
  } else if (mode == kDgrad) {
    // dgrad: B is the transposed weight copy [K, G*N]; scales keep the forward layout
    p.lda = N; p.ldsa = N / 128; p.ldb = (int64_t)G * N; p.ldsb = K / 128;
  } else {
    // wgrad: both operands column-wise with leading dimension ld, one fp32 scale per 128 columns
    p.lda = ld; p.ldsa = ld / 128; p.ldb = ld; p.ldsb = ld / 128;
    p.ld_cols = ld;
  }
  if (mode != kWgrad && M == 0) return ok();
  TRY(check_device());
  return launched(launch_bw_gemm(mode, p, (hipStream_t)stream), fn);
}

mxmoe_status fp8bw_grouped_gemm_fwd(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                    const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                    mxmoe_dtype ydt, void* stream) {
  return bw_gemm_common(kFwd, "fp8bw_grouped_gemm_fwd", kFeedPrecise, qx, sx, qw, sw, offs, G, M, N, K, y, (int)ydt,
                        stream);
}

mxmoe_status fp8bw_grouped_gemm_fwd_fp8feed(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                            const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                            mxmoe_dtype ydt, void* stream) {
  return bw_gemm_common(kFwd, "fp8bw_grouped_gemm_fwd_fp8feed", kFeedFast, qx, sx, qw, sw, offs, G, M, N, K, y,
                        (int)ydt, stream);
}

// Blockwise forward / dgrad with power-of-two scales on the MX kernel (the scale's exponent byte is its
// E8M0 form): fp32 scale rows are K/32 (A: L/32) bytes long, so the MX kernel's byte strides apply.
static mxmoe_status bw_pow2_common(int mode, const char* fn, int feed, const uint8_t* a, const float* sa,
                                   const uint8_t* b, const float* sb, const int32_t* offs, int32_t G, int64_t M,
                                   int64_t N, int64_t K, void* out, int dt, void* stream) {
  TRY(check_gemm_common(fn, offs, G, M, N, K, out, dt));
  TRY(check_ptr(fn, "A operand", a, 16));
  TRY(check_ptr(fn, "A scales", sa, 4));
  TRY(check_ptr(fn, "B operand", b, 16));
  TRY(check_ptr(fn, "B scales", sb, 4));
  GemmArgs p;
  memset(&p, 0, sizeof p);
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.offs = offs; p.out = out;
  p.M = M; p.N = N; p.K = K; p.G = G;
  p.out_bf16 = dt == MXMOE_BF16;
  p.feed = feed;
  p.bw_pow2 = 1;
  p.a_kstride = p.b_kstride = 128;
  if (mode == kFwd) {
    p.lda = K; p.ldsa = K / 32; p.ldb = K; p.ldsb = K / 32;
  } else {
    // B is the transposed weight copy [K, G*N]; its block scales keep the forward layout
    p.lda = N; p.ldsa = N / 32; p.ldb = (int64_t)G * N; p.ldsb = K / 32;
  }
  TRY(check_strides(fn, p, 256));
  if (M == 0) return ok();
  TRY(check_device());
  return launched(launch_mx_gemm(mode, p, (hipStream_t)stream), fn);
}

mxmoe_status fp8bw_grouped_gemm_fwd_pow2(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                         const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* y,
                                         mxmoe_dtype ydt, void* stream) {
  return bw_pow2_common(kFwd, "fp8bw_grouped_gemm_fwd_pow2", kFeedPrecise, qx, sx, qw, sw, offs, G, M, N, K, y,
                        (int)ydt, stream);
}

mxmoe_status fp8bw_grouped_gemm_fwd_pow2_fp8feed(const uint8_t* qx, const float* sx, const uint8_t* qw,
                                                 const float* sw, const int32_t* offs, int32_t G, int64_t M,
                                                 int64_t N, int64_t K, void* y, mxmoe_dtype ydt, void* stream) {
  return bw_pow2_common(kFwd, "fp8bw_grouped_gemm_fwd_pow2_fp8feed", kFeedFast, qx, sx, qw, sw, offs, G, M, N, K, y,
                        (int)ydt, stream);
}

mxmoe_status fp8bw_grouped_gemm_dgrad_pow2(const uint8_t* qdy, const float* sdy, const uint8_t* qwT,
                                           const float* sw, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                           int64_t K, void* dx, mxmoe_dtype dxdt, void* stream) {
  return bw_pow2_common(kDgrad, "fp8bw_grouped_gemm_dgrad_pow2", kFeedPrecise, qdy, sdy, qwT, sw, offs, G, M, N, K,
                        dx, (int)dxdt, stream);
}

mxmoe_status fp8bw_grouped_gemm_dgrad_pow2_fp8feed(const uint8_t* qdy, const float* sdy, const uint8_t* qwT,
                                                   const float* sw, const int32_t* offs, int32_t G, int64_t M,
                                                   int64_t N, int64_t K, void* dx, mxmoe_dtype dxdt, void* stream) {
  return bw_pow2_common(kDgrad, "fp8bw_grouped_gemm_dgrad_pow2_fp8feed", kFeedFast, qdy, sdy, qwT, sw, offs, G, M, N,
                        K, dx, (int)dxdt, stream);
}

static mxmoe_status fp8bw_grouped_gemm_wgrad_pow2_impl(const char* fn, int feed, const uint8_t* qdyT, const float* sdyT,
                                                const uint8_t* qxT, const float* sxT, int64_t ld, const int32_t* offs,
                                                int32_t G, int64_t M, int64_t N, int64_t K, void* dw, int dt,
                                                void* stream) {
  if (G >= 1 && M >= 0 && (ld % 128 || ld < fp8bw_colwise_ld_min(M, G)))
    return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld must be a multiple of 128 and >= fp8bw_colwise_ld_min(M, G)=%lld", fn,
                (long long)ld, (long long)fp8bw_colwise_ld_min(M, G));
  TRY(check_gemm_common(fn, offs, G, M, N, K, dw, dt));
  TRY(check_ptr(fn, "A operand", qdyT, 16));
  TRY(check_ptr(fn, "A scales", sdyT, 4));
  TRY(check_ptr(fn, "B operand", qxT, 16));
  TRY(check_ptr(fn, "B scales", sxT, 4));
  GemmArgs p;
  memset(&p, 0, sizeof p);
  p.a = qdyT; p.sa = sdyT; p.b = qxT; p.sb = sxT; p.offs = offs; p.out = dw;
  p.M = M; p.N = N; p.K = K; p.G = G;
  p.out_bf16 = dt == MXMOE_BF16;
  p.feed = feed;
  p.bw_pow2 = 1;
  p.a_kstride = p.b_kstride = 128;
  // fp32 scale rows of ld / 128 floats = ld / 32 bytes, the MX kernel's byte stride
  p.lda = ld; p.ldsa = ld / 32; p.ldb = ld; p.ldsb = ld / 32;
  p.ld_cols = ld;
  TRY(check_strides(fn, p, 256));
  TRY(check_device());
  return launched(launch_mx_gemm(kWgrad, p, (hipStream_t)stream), fn);
}

mxmoe_status fp8bw_grouped_gemm_wgrad_pow2(const uint8_t* qdyT, const float* sdyT, const uint8_t* qxT,
                                           const float* sxT, int64_t ld, const int32_t* offs, int32_t G, int64_t M,
                                           int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt, void* stream) {
  return fp8bw_grouped_gemm_wgrad_pow2_impl("fp8bw_grouped_gemm_wgrad_pow2", kFeedPrecise, qdyT, sdyT, qxT, sxT, ld,
                                            offs, G, M, N, K, dw, (int)dwdt, stream);
}

mxmoe_status fp8bw_grouped_gemm_wgrad_pow2_fp8feed(const uint8_t* qdyT, const float* sdyT, const uint8_t* qxT,
                                                   const float* sxT, int64_t ld, const int32_t* offs, int32_t G,
                                                   int64_t M, int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt,
                                                   void* stream) {
  return fp8bw_grouped_gemm_wgrad_pow2_impl("fp8bw_grouped_gemm_wgrad_pow2_fp8feed", kFeedFast, qdyT, sdyT, qxT, sxT,
                                            ld, offs, G, M, N, K, dw, (int)dwdt, stream);
}

static mxmoe_status bw_wgrad_impl(const char* fn, int feed, const uint8_t* qdyT, const float* sdyT, const uint8_t* qxT,
                                  const float* sxT, int64_t ld, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                  int64_t K, void* dw, mxmoe_dtype dwdt, void* stream) {
  if (G >= 1 && M >= 0 && (ld % 128 || ld < fp8bw_colwise_ld_min(M, G)))
    return fail(MXMOE_ERR_SHAPE, "%s: ld=%lld must be a multiple of 128 and >= fp8bw_colwise_ld_min(M, G)=%lld", fn,
                (long long)ld, (long long)fp8bw_colwise_ld_min(M, G));
  return bw_gemm_common(kWgrad, fn, feed, qdyT, sdyT, qxT, sxT, offs, G, M, N, K, dw, (int)dwdt, stream, ld);
}

mxmoe_status fp8bw_grouped_gemm_wgrad(const uint8_t* qdyT, const float* sdyT, const uint8_t* qxT, const float* sxT,
                                      int64_t ld, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                                      void* dw, mxmoe_dtype dwdt, void* stream) {
  return bw_wgrad_impl("fp8bw_grouped_gemm_wgrad", kFeedPrecise, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw, dwdt,
                       stream);
}

mxmoe_status fp8bw_grouped_gemm_wgrad_fp8feed(const uint8_t* qdyT, const float* sdyT, const uint8_t* qxT,
                                              const float* sxT, int64_t ld, const int32_t* offs, int32_t G, int64_t M,
                                              int64_t N, int64_t K, void* dw, mxmoe_dtype dwdt, void* stream) {
  return bw_wgrad_impl("fp8bw_grouped_gemm_wgrad_fp8feed", kFeedFast, qdyT, sdyT, qxT, sxT, ld, offs, G, M, N, K, dw,
                       dwdt, stream);
}

mxmoe_status fp8bw_grouped_gemm_dgrad(const uint8_t* qdy, const float* sdy, const uint8_t* qwT, const float* sw,
                                      const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* dx,
                                      mxmoe_dtype dxdt, void* stream) {
  return bw_gemm_common(kDgrad, "fp8bw_grouped_gemm_dgrad", kFeedPrecise, qdy, sdy, qwT, sw, offs, G, M, N, K, dx,
                        (int)dxdt, stream);
}

mxmoe_status fp8bw_grouped_gemm_dgrad_fp8feed(const uint8_t* qdy, const float* sdy, const uint8_t* qwT,
                                              const float* sw, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                                              int64_t K, void* dx, mxmoe_dtype dxdt, void* stream) {
  return bw_gemm_common(kDgrad, "fp8bw_grouped_gemm_dgrad_fp8feed", kFeedFast, qdy, sdy, qwT, sw, offs, G, M, N, K,
                        dx, (int)dxdt, stream);
}

mxmoe_status mxmoe_check_offsets(const int32_t* offs, int32_t G, int64_t M, void* stream) {
  const char* fn = "mxmoe_check_offsets";
  if (G < 1) return fail(MXMOE_ERR_SHAPE, "%s: G < 1", fn);
  if (M < 0) return fail(MXMOE_ERR_SHAPE, "%s: M < 0", fn);
  TRY(check_ptr(fn, "offs", offs, 4));
  std::vector<int32_t> h((size_t)G + 1);
  hipError_t e = hipMemcpyAsync(h.data(), offs, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(MXMOE_ERR_HIP, "%s: copy failed: %s", fn, hipGetErrorString(e));
  if (h[0] != 0) return fail(MXMOE_ERR_OFFSETS, "%s: offs[0] = %d, expected 0", fn, h[0]);
  for (int32_t g = 0; g < G; ++g)
    if (h[g + 1] < h[g]) return fail(MXMOE_ERR_OFFSETS, "%s: offs[%d] = %d < offs[%d] = %d", fn, g + 1, h[g + 1], g, h[g]);
  if ((int64_t)h[G] != M) return fail(MXMOE_ERR_OFFSETS, "%s: offs[G] = %d, expected M = %lld", fn, h[G], (long long)M);
  return ok();
}

}  // extern "C"
