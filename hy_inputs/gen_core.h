/*
 * Seeded synthetic-input generator: core arithmetic shared by the host build
 * (gen_host.c, gcc) and the device build (gen_dev.hip, hipcc).
 *
 * This file holds no arithmetic of the MoE layer itself. It only defines how
 * the layer's inputs (activations, weights, packed ternary codes, scales) are
 * drawn, so that the HIP path under test and the fp64 oracle see the same
 * bytes. Both builds must be compiled with -ffp-contract=off: every floating
 * point step below is a plain IEEE-754 add, subtract or multiply (no division,
 * no square root, no libm call), so the host and device produce bit-identical
 * values by construction.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
 *   key     = (seed, stream id)            one stream per tensor
 *   counter = (i_lo, i_hi, 0, 0)           i = element index (or pair index)
 * Gaussians: the Box-Muller transform (Box and Muller, 1958) on two 53-bit
 * uniforms drawn from one Philox block; element 2i takes the cosine branch of
 * block i and element 2i+1 the sine branch. ln, sqrt and sin/cos are evaluated
 * here with fixed-length series and Newton iterations (documented inline),
 * accurate to a few ulp of fp64 and identical on every IEEE machine.
 * Rounding to bf16: fp64 -> fp32 (round to nearest even), then fp32 -> bf16
 * (round to nearest even on the upper 16 bits).
 */
#ifndef HY_INPUTS_GEN_CORE_H
#define HY_INPUTS_GEN_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define GEN_FN __host__ __device__ static inline
#else
#define GEN_FN static inline
#endif

/* ---- Philox4x32-10 ------------------------------------------------------ */
#define GEN_PHILOX_M0 0xD2511F53u
#define GEN_PHILOX_M1 0xCD9E8D57u
#define GEN_PHILOX_W0 0x9E3779B9u
#define GEN_PHILOX_W1 0xBB67AE85u

typedef struct { uint32_t v[4]; } gen_u32x4;

GEN_FN gen_u32x4 gen_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                   uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)GEN_PHILOX_M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)GEN_PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += GEN_PHILOX_W0;
    k1 += GEN_PHILOX_W1;
  }
  gen_u32x4 o;
  o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
  return o;
}

GEN_FN gen_u32x4 gen_block(uint64_t seed, uint32_t stream, uint64_t ctr) {
  /* The 64-bit seed is folded into the first key word; the stream id (one per
   * tensor) is the second key word. */
  uint32_t k0 = (uint32_t)seed ^ (uint32_t)(seed >> 32);
  return gen_philox4x32_10((uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u, k0, stream);
}

/* ---- bit helpers -------------------------------------------------------- */
GEN_FN uint64_t gen_f64_bits(double x) {
  union { double d; uint64_t u; } c; c.d = x; return c.u;
}
GEN_FN double gen_bits_f64(uint64_t u) {
  union { double d; uint64_t u; } c; c.u = u; return c.d;
}
GEN_FN uint32_t gen_f32_bits(float x) {
  union { float f; uint32_t u; } c; c.f = x; return c.u;
}

/* 53-bit uniform in the open interval (0,1): (a + 1/2) * 2^-53. */
GEN_FN double gen_u01_open(uint32_t hi, uint32_t lo) {
  uint64_t a = (((uint64_t)hi << 32) | lo) >> 11;
  return ((double)a + 0.5) * (1.0 / 9007199254740992.0);
}
/* 53-bit uniform in [0,1): a * 2^-53. */
GEN_FN double gen_u01(uint32_t hi, uint32_t lo) {
  uint64_t a = (((uint64_t)hi << 32) | lo) >> 11;
  return (double)a * (1.0 / 9007199254740992.0);
}

/* ---- elementary functions from + - * only ------------------------------- */

/* 1/x for x in [1.5, 2.5] by Newton's iteration r <- r(2 - x r) from r0 = 0.5;
 * the relative error after n steps is at most 0.25^(2^n); 6 steps. */
GEN_FN double gen_recip_1p5_2p5(double x) {
  double r = 0.5;
  for (int i = 0; i < 6; ++i) r = r * (2.0 - x * r);
  return r;
}

/* Natural log of u in (0,1]. u = m 2^e with m in [sqrt(1/2), sqrt(2)); then
 * ln m = 2 atanh(s), s = (m-1)/(m+1), |s| <= 0.1716, summed to s^23. */
GEN_FN double gen_ln(double u) {
  uint64_t b = gen_f64_bits(u);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = gen_bits_f64((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
  if (m > 1.4142135623730951) { m = m * 0.5; e += 1; }
  double f = m - 1.0;
  double s = f * gen_recip_1p5_2p5(2.0 + f);
  double p = s * s;
  double q = 1.0 / 23.0;
  q = 1.0 / 21.0 + p * q;
  q = 1.0 / 19.0 + p * q;
  q = 1.0 / 17.0 + p * q;
  q = 1.0 / 15.0 + p * q;
  q = 1.0 / 13.0 + p * q;
  q = 1.0 / 11.0 + p * q;
  q = 1.0 / 9.0 + p * q;
  q = 1.0 / 7.0 + p * q;
  q = 1.0 / 5.0 + p * q;
  q = 1.0 / 3.0 + p * q;
  q = 1.0 + p * q;
  return (double)e * 0.6931471805599453 + 2.0 * s * q;
}

/* sqrt(x) for x in [2^-60, 2^10]: reciprocal square root by Newton's iteration
 * y <- y(3/2 - x y^2 / 2) from the classic exponent-halving bit estimate
 * (initial relative error < 3.5%), 6 steps, then sqrt = x y. */
GEN_FN double gen_sqrt(double x) {
  double y = gen_bits_f64(0x5FE6EB50C7B537A9ull - (gen_f64_bits(x) >> 1));
  for (int i = 0; i < 6; ++i) y = y * (1.5 - 0.5 * x * y * y);
  return x * y;
}

/* sin and cos of x in [0, pi/4] by Taylor series to x^18 / x^19. */
GEN_FN void gen_sincos_small(double x, double* s, double* c) {
  double p = x * x;
  double ss = 1.0 / 121645100408832000.0;                 /* 1/19! */
  ss = -1.0 / 355687428096000.0 + p * ss;                 /* 1/17! */
  ss = 1.0 / 1307674368000.0 + p * ss;                    /* 1/15! */
  ss = -1.0 / 6227020800.0 + p * ss;                      /* 1/13! */
  ss = 1.0 / 39916800.0 + p * ss;                         /* 1/11! */
  ss = -1.0 / 362880.0 + p * ss;                          /* 1/9!  */
  ss = 1.0 / 5040.0 + p * ss;                             /* 1/7!  */
  ss = -1.0 / 120.0 + p * ss;                             /* 1/5!  */
  ss = 1.0 / 6.0 + p * ss;                                /* 1/3!  */
  *s = x - x * p * ss;
  double cc = 1.0 / 6402373705728000.0;                   /* 1/18! */
  cc = -1.0 / 20922789888000.0 + p * cc;                  /* 1/16! */
  cc = 1.0 / 87178291200.0 + p * cc;                      /* 1/14! */
  cc = -1.0 / 479001600.0 + p * cc;                       /* 1/12! */
  cc = 1.0 / 3628800.0 + p * cc;                          /* 1/10! */
  cc = -1.0 / 40320.0 + p * cc;                           /* 1/8!  */
  cc = 1.0 / 720.0 + p * cc;                              /* 1/6!  */
  cc = -1.0 / 24.0 + p * cc;                              /* 1/4!  */
  cc = 0.5 + p * cc;                                      /* 1/2!  */
  *c = 1.0 - p * cc;
}

/* cos and sin of 2 pi a for a in [0,1): quadrant q = floor(4a), remainder r in
 * [0,1) of a quarter turn, folded to an angle in [0, pi/4]. */
GEN_FN void gen_cossin_turn(double a, double* co, double* si) {
  double a4 = a * 4.0;
  int q = (int)a4;
  double r = a4 - (double)q;
  double s, c;
  if (r <= 0.5) {
    gen_sincos_small(r * 1.5707963267948966, &s, &c);
  } else {
    double t, u;
    gen_sincos_small((1.0 - r) * 1.5707963267948966, &t, &u);
    s = u; c = t;
  }
  switch (q & 3) {
    case 0: *co = c; *si = s; break;
    case 1: *co = -s; *si = c; break;
    case 2: *co = -c; *si = -s; break;
    default: *co = s; *si = -c; break;
  }
}

/* ---- rounding ----------------------------------------------------------- */
GEN_FN uint16_t gen_f32_to_bf16_rne(float f) {
  uint32_t u = gen_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* ---- element generators ------------------------------------------------- */

/* Element i of a Gaussian tensor with the given standard deviation, as bf16. */
GEN_FN uint16_t gen_gauss_bf16_elem(uint64_t seed, uint32_t stream, uint64_t i, double std) {
  gen_u32x4 r = gen_block(seed, stream, i >> 1);
  double u1 = gen_u01_open(r.v[0], r.v[1]);
  double u2 = gen_u01(r.v[2], r.v[3]);
  double rad = gen_sqrt(-2.0 * gen_ln(u1));
  double co, si;
  gen_cossin_turn(u2, &co, &si);
  double z = (i & 1) ? rad * si : rad * co;
  return gen_f32_to_bf16_rne((float)(z * std));
}

/* Element i of a tensor uniform on [lo, lo + width), as bf16. */
GEN_FN uint16_t gen_uniform_bf16_elem(uint64_t seed, uint32_t stream, uint64_t i,
                                      double lo, double width) {
  gen_u32x4 r = gen_block(seed, stream, i);
  double u = gen_u01(r.v[0], r.v[1]);
  return gen_f32_to_bf16_rne((float)(lo + u * width));
}

/* Word i of a tensor of uniformly random 32-bit words. */
GEN_FN uint32_t gen_u32_elem(uint64_t seed, uint32_t stream, uint64_t i) {
  gen_u32x4 r = gen_block(seed, stream, i >> 2);
  return r.v[i & 3];
}

#endif /* HY_INPUTS_GEN_CORE_H */
