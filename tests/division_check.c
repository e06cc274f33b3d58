/* Host check of the blockwise quantisers' element division (precision_moe_expert_mx_amd/csrc/quant_bw.hip).
 *
 * For bf16 amax values with exponent field >= EMIN (every STRIDE-th one) and every bf16 v with
 * |v| <= amax, both signs: the E4M3 code of the IEEE quotient fl32(v / s), s = fl32(amax / 448), must
 * equal the code of the kernels' form q0 = fl32(v y), r = fma(-s, q0, v), q = copysign(fma(r, y, q0), v)
 * with y = fl32(1 / s).  The second form is evaluated twice: with IEEE denormals and with denormals
 * flushed (MXCSR FTZ and DAZ), since the result must not depend on the device's denormal mode.
 * Arguments: EMIN [STRIDE [EMAX [NOSIGN]]]: amax exponent fields [EMIN, EMAX), every STRIDE-th amax;
 * NOSIGN = 1 drops the sign restore (a planted mistake the check must catch).
 * Prints the number of pairs and of code mismatches.  Build: gcc -O2 -mfma division_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

static float bf16(uint32_t bits) { uint32_t b = bits << 16; float x; memcpy(&x, &b, 4); return x; }

/* E4M3 (bias 7, max 448) code of x: nearest, ties to even, saturating, sign kept (also for zero). */
static int e4m3(float x) {
  const int sgn = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  int e = a > 0 ? (int)floor(log2(a)) : -6;
  if (e < -6) e = -6;
  double q = ldexp(1.0, e - 3);                     /* quantum of the binade (subnormal below 2^-6) */
  double v = nearbyint(a / q) * q;                  /* exact: q is a power of two */
  if (v > 448.0) v = 448.0;
  if (v == 0) return sgn;
  int E = (int)floor(log2(v));
  if (E < -6) return sgn | (int)(v / ldexp(1.0, -9));
  return sgn | ((E + 7) << 3) | ((int)(v / ldexp(1.0, E - 3)) - 8);
}

static int nosign;

static float kernel_quot(float v, float s, float y) {
  volatile float vv = v;                            /* keep the evaluation under the current MXCSR */
  float q0 = vv * y;
  float r = fmaf(-s, q0, vv);
  float q = fmaf(r, y, q0);
  return nosign ? q : copysignf(q, vv);
}

static unsigned char ref[2][32768];

int main(int argc, char** argv) {
  const int emin = argc > 1 ? atoi(argv[1]) : 68;
  const int stride = argc > 2 ? atoi(argv[2]) : 1;
  const uint32_t emax = argc > 3 ? (uint32_t)atoi(argv[3]) : 255;
  nosign = argc > 4 ? atoi(argv[4]) : 0;
  const unsigned csr = _mm_getcsr();
  long long pairs = 0, bad = 0;
  for (uint32_t am = (uint32_t)emin << 7; am < (emax << 7) && am < 0x7F80; am += stride) {
    const float s = bf16(am) / 448.0f;
    volatile float one = 1.0f;
    const float y = one / s;
    for (uint32_t vb = 0; vb <= am; ++vb)
      for (int sg = 0; sg < 2; ++sg) ref[sg][vb] = (unsigned char)e4m3(bf16(vb | (sg ? 0x8000u : 0)) / s);
    for (int ftz = 0; ftz < 2; ++ftz)
      for (uint32_t vb = 0; vb <= am; ++vb)
        for (int sg = 0; sg < 2; ++sg) {
          if (ftz) _mm_setcsr(csr | 0x8040);
          float q = kernel_quot(bf16(vb | (sg ? 0x8000u : 0)), s, y);
          _mm_setcsr(csr);
          uint32_t qb;
          memcpy(&qb, &q, 4);
          if (ftz && (qb & 0x7F800000u) == 0) qb &= 0x80000000u;   /* a flushed result is a signed zero */
          memcpy(&q, &qb, 4);
          ++pairs;
          bad += e4m3(q) != ref[sg][vb];
        }
  }
  printf("%lld %lld\n", pairs, bad);
  return 0;
}
