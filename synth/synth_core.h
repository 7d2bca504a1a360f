/*
 * synth_core.h - seeded, counter-based synthetic inputs.
 *
 * This header is the one piece shared by the host generator (synth_host.c,
 * built with gcc), the device generator (synth_device.hip, built with hipcc)
 * and through them by both the CPU oracle and the GPU path.  It holds none of
 * the attention method's arithmetic: only a random-number generator and the
 * mapping of its output onto N(0,1) values.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11): a 4x32-bit counter, a 2x32-bit key,
 * ten rounds of two 32x32->64 multiplies with xor mixing, and a Weyl-sequence
 * key schedule.  Element e of tensor `tid` under seed `s` is normal number
 * (e mod 4) of the block at counter (e/4 low word, e/4 high word, tid, 0)
 * under key (s low word, s high word).  Every element can be generated on its
 * own (random access), so a slab or a single chunk of a huge tensor is
 * regenerated without generating the rest.
 *
 * Normals: Box-Muller on pairs of 32-bit words, u = (w + 0.5) * 2^-32 in (0,1),
 * z0 = r cos(2 pi u2), z1 = r sin(2 pi u2), r = sqrt(-2 ln u1).  The logarithm,
 * sine and cosine below are written out in plain double arithmetic (an
 * atanh-series logarithm after exponent extraction, Taylor series for sine and
 * cosine on a quarter period after exact quadrant reduction), so that host and
 * device produce bit-identical values.  Every file that includes this header
 * must be compiled with floating-point contraction turned off; the pragma
 * below enforces that for clang, the build line does so for gcc.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <math.h>
#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#if defined(__clang__)
#pragma clang fp contract(off)
#endif

/* Philox4x32 round constants from the SC'11 paper. */
#define SYNTH_PHILOX_M0 0xD2511F53u
#define SYNTH_PHILOX_M1 0xCD9E8D57u
#define SYNTH_PHILOX_W0 0x9E3779B9u
#define SYNTH_PHILOX_W1 0xBB67AE85u

SYNTH_FN void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                  uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += SYNTH_PHILOX_W0;
      k1 += SYNTH_PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)SYNTH_PHILOX_M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)SYNTH_PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

SYNTH_FN double synth_bits_to_double(uint64_t b) {
  double x;
  memcpy(&x, &b, sizeof x);
  return x;
}

SYNTH_FN uint64_t synth_double_to_bits(double x) {
  uint64_t b;
  memcpy(&b, &x, sizeof b);
  return b;
}

/* Natural logarithm of a normal, positive double.  x = m * 2^e with m in
 * [sqrt(1/2), sqrt(2)); ln m = 2 atanh(s), s = (m-1)/(m+1), |s| < 0.1716,
 * summed to the s^23 term (truncation below 1e-18 relative). */
SYNTH_FN double synth_log(double x) {
  const double ln2 = 0.69314718055994530942;
  const double sqrt_half = 0.70710678118654752440;
  uint64_t b = synth_double_to_bits(x);
  int e = (int)((b >> 52) & 0x7ff) - 1022;
  double m = synth_bits_to_double((b & 0x000fffffffffffffull) | 0x3fe0000000000000ull);
  if (m < sqrt_half) {
    m = m * 2.0;
    e -= 1;
  }
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  /* 1/(2j+1), j = 11 .. 0 */
  const double inv_odd[12] = {1.0 / 23.0, 1.0 / 21.0, 1.0 / 19.0, 1.0 / 17.0,
                              1.0 / 15.0, 1.0 / 13.0, 1.0 / 11.0, 1.0 / 9.0,
                              1.0 / 7.0,  1.0 / 5.0,  1.0 / 3.0,  1.0};
  double p = inv_odd[0];
  for (int j = 1; j < 12; ++j) p = p * s2 + inv_odd[j];
  return (double)e * ln2 + 2.0 * s * p;
}

/* sin and cos of a in [0, pi/2), Taylor series to the a^25 / a^24 terms. */
SYNTH_FN void synth_sincos_quarter(double a, double* sn, double* cs) {
  /* sin a = a (1 - a^2/(2*3) (1 - a^2/(4*5) (...))), cos a likewise with
   * (1*2), (3*4), ...; the reciprocals are folded at compile time. */
  const double inv_s[12] = {1.0 / (24.0 * 25.0), 1.0 / (22.0 * 23.0), 1.0 / (20.0 * 21.0),
                            1.0 / (18.0 * 19.0), 1.0 / (16.0 * 17.0), 1.0 / (14.0 * 15.0),
                            1.0 / (12.0 * 13.0), 1.0 / (10.0 * 11.0), 1.0 / (8.0 * 9.0),
                            1.0 / (6.0 * 7.0),   1.0 / (4.0 * 5.0),   1.0 / (2.0 * 3.0)};
  const double inv_c[12] = {1.0 / (23.0 * 24.0), 1.0 / (21.0 * 22.0), 1.0 / (19.0 * 20.0),
                            1.0 / (17.0 * 18.0), 1.0 / (15.0 * 16.0), 1.0 / (13.0 * 14.0),
                            1.0 / (11.0 * 12.0), 1.0 / (9.0 * 10.0),  1.0 / (7.0 * 8.0),
                            1.0 / (5.0 * 6.0),   1.0 / (3.0 * 4.0),   1.0 / (1.0 * 2.0)};
  double a2 = a * a;
  double ps = 1.0, pc = 1.0;
  for (int j = 0; j < 12; ++j) {
    ps = 1.0 - (ps * a2) * inv_s[j];
    pc = 1.0 - (pc * a2) * inv_c[j];
  }
  *sn = a * ps;
  *cs = pc;
}

/* Two standard normals from two 32-bit words. */
SYNTH_FN void synth_box_muller(uint32_t w1, uint32_t w2, double* z0, double* z1) {
  const double two_m32 = 2.3283064365386962890625e-10; /* 2^-32 */
  const double half_pi = 1.57079632679489661923;
  double u1 = ((double)w1 + 0.5) * two_m32;
  double u2 = ((double)w2 + 0.5) * two_m32;
  double r = sqrt(-2.0 * synth_log(u1));
  double v = u2 * 4.0; /* exact */
  int q = (int)v;      /* quadrant 0..3 */
  double f = v - (double)q;
  double sn, cs;
  synth_sincos_quarter(f * half_pi, &sn, &cs);
  double c, s;
  switch (q & 3) {
    case 0: c = cs; s = sn; break;
    case 1: c = -sn; s = cs; break;
    case 2: c = -cs; s = -sn; break;
    default: c = sn; s = -cs; break;
  }
  *z0 = r * c;
  *z1 = r * s;
}

/* Elements 4*blk .. 4*blk+3 of tensor `tid` under `seed`: four standard
 * normals (double). */
SYNTH_FN void synth_normal4(uint64_t seed, uint32_t tid, uint64_t blk, double z[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), tid, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  synth_philox4x32_10(ctr, key, w);
  synth_box_muller(w[0], w[1], &z[0], &z[1]);
  synth_box_muller(w[2], w[3], &z[2], &z[3]);
}

/* Element e of tensor `tid` under `seed`: a standard normal (double). */
SYNTH_FN double synth_normal(uint64_t seed, uint32_t tid, uint64_t e) {
  double z[4];
  synth_normal4(seed, tid, e >> 2, z);
  return z[e & 3u];
}

/* Round-to-nearest-even of a float to bfloat16 bits (no NaN inputs). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7fffu + lsb;
  return (uint16_t)(b >> 16);
}

/* Uniform integer in [lo, hi] from word w (multiply-shift). */
SYNTH_FN int64_t synth_uniform_int(uint32_t w, int64_t lo, int64_t hi) {
  uint64_t span = (uint64_t)(hi - lo + 1);
  return lo + (int64_t)(((uint64_t)w * span) >> 32);
}

/* The first word of the block at counter (i, 0, tid, 0x5eed). */
SYNTH_FN uint32_t synth_word(uint64_t seed, uint32_t tid, uint64_t i) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), tid, 0x5eedu};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  synth_philox4x32_10(ctr, key, w);
  return w[0];
}

#endif /* SYNTH_CORE_H */
