/*
 * Seeded synthetic inputs, host side.
 *
 * Counter-based generator: Philox4x32 with 10 rounds, as defined by Salmon,
 * Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
 * (SC'11, section 3.2): a 4x32-bit counter is passed through 10 rounds, each
 * round multiplying words 0 and 2 by the constants 0xD2511F53 and 0xCD9E8D57,
 * mixing the high halves with the other two words and the 2x32-bit key, and
 * permuting; the key is bumped by the Weyl constants 0x9E3779B9 / 0xBB67AE85
 * between rounds.
 *
 * Element n of a tensor stream (key0, key1) uses counter (n_lo, n_hi, 0, 0).
 * Its words give one standard normal draw by the Box-Muller transform (G. E. P.
 * Box and M. E. Muller, "A note on the generation of random normal deviates",
 * Ann. Math. Statist. 29, 1958): z = sqrt(-2 ln u1) cos(2 pi u2), with u1 in
 * (0, 1] from the top 53 bits of words 0-1 and u2 in [0, 1) from word 2.  The
 * draw is scaled by sigma in double, rounded to fp32 (RNE) and, for bf16
 * tensors, from fp32 to bf16 (RNE).
 *
 * The logarithm, square root and cosine are written out here from +, -, *, /
 * only (series and Newton steps), each an IEEE double operation rounded on its
 * own (built with -ffp-contract=off, so none is fused), and the device fill
 * (fill_device.hip) performs the same operations in the same order: both sides
 * produce the same bits for every element.
 *
 * This module holds no arithmetic of the decode layer itself.
 */
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k0;
  uint32_t n2 = hi0 ^ c[3] ^ k1;
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

static inline void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    philox_round(c, k0, k1);
  }
}

/* Raw block function, exported for known-answer tests. */
void synth_philox4x32_10(const uint32_t in[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4];
  memcpy(c, in, sizeof c);
  philox10(c, key[0], key[1]);
  memcpy(out, c, sizeof c);
}

/* Series coefficients (hex literals, so both compilers hold the same doubles):
 * ln m = 2 s sum_j s^2j / (2j + 1) with s = (m - 1) / (m + 1);
 * sin x = x sum_j (-1)^j x^2j / (2j + 1)!, cos x = sum_j (-1)^j x^2j / (2j)!. */
static const double kAtanh[12] = {
    0x1.0000000000000p+0, 0x1.5555555555555p-2, 0x1.999999999999ap-3, 0x1.2492492492492p-3,
    0x1.c71c71c71c71cp-4, 0x1.745d1745d1746p-4, 0x1.3b13b13b13b14p-4, 0x1.1111111111111p-4,
    0x1.e1e1e1e1e1e1ep-5, 0x1.af286bca1af28p-5, 0x1.8618618618618p-5, 0x1.642c8590b2164p-5};
static const double kSin[11] = {
    0x1.0000000000000p+0, -0x1.5555555555555p-3, 0x1.1111111111111p-7, -0x1.a01a01a01a01ap-13,
    0x1.71de3a556c734p-19, -0x1.ae64567f544e4p-26, 0x1.6124613a86d09p-33, -0x1.ae7f3e733b81fp-41,
    0x1.952c77030ad4ap-49, -0x1.2f49b46814157p-57, 0x1.71b8ef6dcf572p-66};
static const double kCos[12] = {
    0x1.0000000000000p+0, -0x1.0000000000000p-1, 0x1.5555555555555p-5, -0x1.6c16c16c16c17p-10,
    0x1.a01a01a01a01ap-16, -0x1.27e4fb7789f5cp-22, 0x1.1eed8eff8d898p-29, -0x1.93974a8c07c9dp-37,
    0x1.ae7f3e733b81fp-45, -0x1.6827863b97d97p-53, 0x1.e542ba4020225p-62, -0x1.0ce396db7f853p-70};
#define LN2 0x1.62e42fefa39efp-1
#define SQRT2 0x1.6a09e667f3bcdp+0
#define HALF_PI 0x1.921fb54442d18p+0

static inline double bits_to_f64(uint64_t b) {
  double d;
  memcpy(&d, &b, 8);
  return d;
}
static inline uint64_t f64_to_bits(double d) {
  uint64_t b;
  memcpy(&b, &d, 8);
  return b;
}

/* ln u for u in [2^-53, 1]: u = 2^e m with m in [sqrt(1/2), sqrt(2)), then the atanh series
 * to s^23 (|s| < 0.172: the first term left out is below 1e-18 of the result). */
static inline double ln_unit(double u) {
  const uint64_t b = f64_to_bits(u);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = bits_to_f64((b & 0xFFFFFFFFFFFFFull) | (1023ull << 52));
  if (m > SQRT2) {
    m = m * 0.5;
    e += 1;
  }
  const double s = (m - 1.0) / (m + 1.0);
  const double s2 = s * s;
  double p = kAtanh[11];
  for (int j = 10; j >= 0; --j) p = p * s2 + kAtanh[j];
  return (double)e * LN2 + 2.0 * s * p;
}

/* sqrt a for a >= 0: a first guess from the halved exponent bits (within 6.1%), then four
 * Newton steps (relative error 6.1e-2 -> 1.9e-3 -> 1.8e-6 -> 1.6e-12 -> 1.3e-24). */
static inline double sqrt_newton(double a) {
  if (a == 0.0) return 0.0;
  double y = bits_to_f64((f64_to_bits(a) >> 1) + 0x1FF8000000000000ull);
  for (int i = 0; i < 4; ++i) y = 0.5 * (y + a / y);
  return y;
}

/* cos(2 pi w / 2^32): quarter turn q from the top two bits, x in [0, pi/2) from the rest;
 * cos(q pi/2 + x) is cos x, -sin x, -cos x, sin x for q = 0..3.  Series to x^21 (sine) and
 * x^22 (cosine): the first term left out is below 1.3e-18. */
static inline double cos_turn(uint32_t w) {
  const uint32_t q = w >> 30;
  const double x = (double)(w & 0x3FFFFFFFu) * 0x1p-30 * HALF_PI;
  const double x2 = x * x;
  double v;
  if (q & 1u) {
    double p = kSin[10];
    for (int j = 9; j >= 0; --j) p = p * x2 + kSin[j];
    v = x * p;
  } else {
    double p = kCos[11];
    for (int j = 10; j >= 0; --j) p = p * x2 + kCos[j];
    v = p;
  }
  return (q == 1 || q == 2) ? -v : v;
}

static inline float element_f32(uint64_t n, uint32_t key0, uint32_t key1, double sigma) {
  uint32_t c[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
  philox10(c, key0, key1);
  const uint64_t m53 = (((uint64_t)c[0] << 32) | c[1]) >> 11;
  const double u1 = (double)(m53 + 1ull) * 0x1p-53;
  const double r = sqrt_newton(-2.0 * ln_unit(u1));
  const double v = r * cos_turn(c[2]) * sigma;
  return (float)v;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* dtype 0: fp32 output, dtype 1: bf16 bits (uint16). Elements first..first+count-1. */
void synth_fill(void* out, int dtype, uint64_t first, uint64_t count, uint32_t key0,
                uint32_t key1, double sigma) {
  if (dtype == 0) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i) o[i] = element_f32(first + (uint64_t)i, key0, key1, sigma);
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i)
      o[i] = f32_to_bf16_rne(element_f32(first + (uint64_t)i, key0, key1, sigma));
  }
}

/* Raw first output word of element n: uniform 32-bit integers (used for permutations). */
void synth_u32(uint32_t* out, uint64_t first, uint64_t count, uint32_t key0, uint32_t key1) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i) {
    uint64_t n = first + (uint64_t)i;
    uint32_t c[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
    philox10(c, key0, key1);
    out[i] = c[0];
  }
}
