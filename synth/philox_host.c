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
 * Its four output words are summed (Irwin-Hall with 4 terms), centred, and
 * scaled in double precision; the result is rounded to fp32 (RNE) and, for
 * bf16 tensors, from fp32 to bf16 (RNE).  Every step is integer or a single
 * IEEE operation, so the device fill (fill_device.hip) produces the same bits.
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

static inline float element_f32(uint64_t n, uint32_t key0, uint32_t key1, double scale) {
  uint32_t c[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
  philox10(c, key0, key1);
  uint64_t s = (uint64_t)c[0] + c[1] + c[2] + c[3];
  int64_t centred = (int64_t)s - (int64_t)((1ull << 33) - 2ull);
  double v = (double)centred * scale;
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
                uint32_t key1, double scale) {
  if (dtype == 0) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i) o[i] = element_f32(first + (uint64_t)i, key0, key1, scale);
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i)
      o[i] = f32_to_bf16_rne(element_f32(first + (uint64_t)i, key0, key1, scale));
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
