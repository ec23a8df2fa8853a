/*
 * Seeded synthetic inputs: one counter-based generator, compiled twice.
 *
 * This header is included by synth_cpu.c (gcc, host) and synth_gpu.hip (hipcc,
 * gfx950).  Both builds must produce the same bits for the same arguments, so
 * the arithmetic below uses only IEEE-754 double +, -, *, / and sqrt (all
 * correctly rounded on both sides) with floating-point contraction disabled
 * (-ffp-contract=off on both compile lines); no libm call is made.
 *
 * It holds no arithmetic of the MoE layer itself: it only draws numbers.
 *
 * Generator: Philox4x32-10, as published by Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): 10 rounds of the
 * 4x32 Philox S-box with multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key
 * increments 0x9E3779B9 / 0xBB67AE85.
 *
 * Stream layout.  A value is addressed by (seed, tag, layer, expert, matrix,
 * index i).  Key = (seed, tag); counter = (j lo32, j hi32, expert | matrix<<16,
 * layer) with j = i / 4; the four 32-bit outputs give the four normals
 * 4j .. 4j+3 by two Box-Muller pairs: (r0, r1) -> z0 = R(r0) cos(theta(r1)),
 * z1 = R(r0) sin(theta(r1)); (r2, r3) -> z2, z3.  R(r) = sqrt(-2 ln u) with
 * u = (r + 1) * 2^-32 in (0, 1]; theta(r) = 2 pi r 2^-32.  The fp32 value is
 * the double z * sigma rounded to nearest-even.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H
#include <stdint.h>

#ifdef __HIPCC__
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_PHILOX_M0 0xD2511F53u
#define SYN_PHILOX_M1 0xCD9E8D57u
#define SYN_PHILOX_W0 0x9E3779B9u
#define SYN_PHILOX_W1 0xBB67AE85u

enum {
  SYN_TAG_X = 1,      /* token activations */
  SYN_TAG_ROUTER = 2, /* router weights */
  SYN_TAG_EXPERT = 3, /* expert weights (matrix 0 gate, 1 up, 2 down) */
  SYN_TAG_CALIB = 4,  /* calibration batch */
  SYN_TAG_ZIPF = 5    /* expert popularity permutation */
};

typedef struct { uint32_t v[4]; } syn_u32x4;

SYN_FN syn_u32x4 syn_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                   uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += SYN_PHILOX_W0; k1 += SYN_PHILOX_W1; }
    uint64_t p0 = (uint64_t)SYN_PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)SYN_PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  syn_u32x4 o;
  o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
  return o;
}

/* ln(u), u = (r + 1) 2^-32, from ln u = e ln2 + ln m with m in (1/sqrt2, sqrt2]
 * and ln m = 2 atanh(s), s = (m - 1)/(m + 1), |s| <= 0.1716, by its odd series
 * through s^25 (truncation below 1e-17). */
SYN_FN double syn_ln_unit(uint32_t r) {
  uint64_t n = (uint64_t)r + 1u;                 /* 1 .. 2^32 */
  int e = 63 - __builtin_clzll(n);               /* floor(log2 n) */
  double m = (double)n / (double)(1ull << e);    /* [1, 2), exact */
  if (m > 1.4142135623730951) { m = m * 0.5; e += 1; }
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  double p = 1.0 / 25.0;
  p = p * s2 + 1.0 / 23.0;
  p = p * s2 + 1.0 / 21.0;
  p = p * s2 + 1.0 / 19.0;
  p = p * s2 + 1.0 / 17.0;
  p = p * s2 + 1.0 / 15.0;
  p = p * s2 + 1.0 / 13.0;
  p = p * s2 + 1.0 / 11.0;
  p = p * s2 + 1.0 / 9.0;
  p = p * s2 + 1.0 / 7.0;
  p = p * s2 + 1.0 / 5.0;
  p = p * s2 + 1.0 / 3.0;
  p = p * s2 + 1.0;
  return (double)(e - 32) * 0.6931471805599453 + 2.0 * s * p;
}

/* cos and sin of 2 pi r 2^-32: quadrant from the top two bits, then Taylor
 * series of the remaining angle a in [0, pi/2) through a^23 / a^24. */
SYN_FN void syn_cossin_turn(uint32_t r, double* c, double* s) {
  uint32_t q = r >> 30;
  double a = (double)(r & 0x3FFFFFFFu) * (1.5707963267948966 / 1073741824.0);
  double a2 = a * a;
  double sn = 1.0 - a2 / 506.0;
  sn = 1.0 - a2 / 420.0 * sn;
  sn = 1.0 - a2 / 342.0 * sn;
  sn = 1.0 - a2 / 272.0 * sn;
  sn = 1.0 - a2 / 210.0 * sn;
  sn = 1.0 - a2 / 156.0 * sn;
  sn = 1.0 - a2 / 110.0 * sn;
  sn = 1.0 - a2 / 72.0 * sn;
  sn = 1.0 - a2 / 42.0 * sn;
  sn = 1.0 - a2 / 20.0 * sn;
  sn = 1.0 - a2 / 6.0 * sn;
  sn = a * sn;
  double cs = 1.0 - a2 / 552.0;
  cs = 1.0 - a2 / 462.0 * cs;
  cs = 1.0 - a2 / 380.0 * cs;
  cs = 1.0 - a2 / 306.0 * cs;
  cs = 1.0 - a2 / 240.0 * cs;
  cs = 1.0 - a2 / 182.0 * cs;
  cs = 1.0 - a2 / 132.0 * cs;
  cs = 1.0 - a2 / 90.0 * cs;
  cs = 1.0 - a2 / 56.0 * cs;
  cs = 1.0 - a2 / 30.0 * cs;
  cs = 1.0 - a2 / 12.0 * cs;
  cs = 1.0 - a2 / 2.0 * cs;
  switch (q) {
    case 0: *c = cs; *s = sn; break;
    case 1: *c = -sn; *s = cs; break;
    case 2: *c = -cs; *s = -sn; break;
    default: *c = sn; *s = -cs; break;
  }
}

/* Four consecutive N(0, sigma^2) values 4j .. 4j+3 of one stream, as fp32. */
SYN_FN void syn_normal4(uint32_t seed, uint32_t tag, uint32_t layer, uint32_t expert,
                        uint32_t matrix, uint64_t j, double sigma, float out[4]) {
  syn_u32x4 r = syn_philox4x32_10((uint32_t)j, (uint32_t)(j >> 32),
                                  (expert & 0xFFFFu) | (matrix << 16), layer, seed, tag);
  for (int h = 0; h < 2; ++h) {
    double rad = __builtin_sqrt(-2.0 * syn_ln_unit(r.v[2 * h]));
    double c, s;
    syn_cossin_turn(r.v[2 * h + 1], &c, &s);
    out[2 * h] = (float)(rad * c * sigma);
    out[2 * h + 1] = (float)(rad * s * sigma);
  }
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
SYN_FN uint16_t syn_f32_to_bf16(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  u = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif
