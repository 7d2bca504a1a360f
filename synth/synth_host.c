/*
 * synth_host.c - host side of the seeded input generator (see synth_core.h).
 * Built with gcc -ffp-contract=off -fopenmp into libsynth_host.so.
 */
#include <stdint.h>
#include <stdlib.h>

#include "synth_core.h"

/* dtype codes shared with the Python wrapper. */
enum { SYNTH_F32 = 0, SYNTH_BF16 = 1, SYNTH_F64 = 2 };

/* Fill out[i] = round(scale * N(0,1)) for elements first .. first+n-1 of
 * tensor `tid`.  Returns 0, or -1 for an unknown dtype. */
int synth_fill_normal(void* out, int dtype, uint64_t first, uint64_t n, uint64_t seed,
                      uint32_t tid, double scale) {
  if (dtype != SYNTH_F32 && dtype != SYNTH_BF16 && dtype != SYNTH_F64) return -1;
  if (n == 0) return 0;
  /* Work in whole Philox blocks of four elements; blocks that straddle the
   * requested range write only their elements inside it. */
  const int64_t b0 = (int64_t)(first >> 2);
  const int64_t b1 = (int64_t)((first + n - 1) >> 2);
#pragma omp parallel for schedule(static)
  for (int64_t b = b0; b <= b1; ++b) {
    double z[4];
    synth_normal4(seed, tid, (uint64_t)b, z);
    for (int j = 0; j < 4; ++j) {
      uint64_t e = (uint64_t)b * 4u + (uint64_t)j;
      if (e < first || e >= first + n) continue;
      uint64_t i = e - first;
      double v = scale * z[j];
      if (dtype == SYNTH_F32)
        ((float*)out)[i] = (float)v;
      else if (dtype == SYNTH_BF16)
        ((uint16_t*)out)[i] = synth_f32_to_bf16((float)v);
      else
        ((double*)out)[i] = v;
    }
  }
  return 0;
}

/* Raw Philox4x32-10 block, exposed for known-answer tests. */
void synth_philox_block(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  synth_philox4x32_10(ctr, key, out);
}

/* The generator's own log / sincos, exposed so tests can check them
 * against libm. */
double synth_log_host(double x) { return synth_log(x); }
void synth_sincos_quarter_host(double a, double* s, double* c) { synth_sincos_quarter(a, s, c); }

/* Variable chunk lengths: i.i.d. uniform integers in [lo, hi] (word i of
 * tensor `tid`), drawn until their sum reaches L; the last one is cut so the
 * sum is exactly L.  Writes offsets[0..n] with offsets[0] = 0, offsets[n] = L
 * and returns n, or -1 if more than max_chunks would be needed. */
int64_t synth_chunk_offsets(int32_t* offsets, int64_t max_chunks, int64_t L, int64_t lo,
                            int64_t hi, uint64_t seed, uint32_t tid) {
  if (lo < 1 || hi < lo || L < 0) return -1;
  int64_t n = 0, pos = 0;
  offsets[0] = 0;
  while (pos < L) {
    if (n >= max_chunks) return -1;
    int64_t len = synth_uniform_int(synth_word(seed, tid, (uint64_t)n), lo, hi);
    if (pos + len > L) len = L - pos;
    pos += len;
    ++n;
    offsets[n] = (int32_t)pos;
  }
  return n;
}

/* A uniform index in [0, n) (word 0 of tensor `tid`); used to place a planted
 * needle chunk. */
int64_t synth_pick_index(int64_t n, uint64_t seed, uint32_t tid) {
  if (n <= 0) return -1;
  return synth_uniform_int(synth_word(seed, tid, 0), 0, n - 1);
}
