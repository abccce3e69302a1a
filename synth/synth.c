/*
 * Seeded synthetic inputs for the Attention Residuals operator.
 *
 * This file holds no part of the operator's arithmetic: it only draws numbers.
 * Both the HIP path (through a host-to-device copy) and the fp64 oracle read
 * what it writes, so the two sides see bit-identical inputs.
 *
 * Generator: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * counter, i.e. value(c) = mix64(key + (c + 1) * GOLDEN_GAMMA).  Every value is
 * a pure function of (seed, stream, counter), so any token range of any tensor
 * can be regenerated on its own, in any order and on any number of threads.
 *
 * Normal variates: Box-Muller (Box and Muller, 1958) on one 64-bit draw split
 * into two 24-bit uniforms in (0, 1); counter 2p yields the cosine branch and
 * counter 2p+1 the sine branch of pair p.  log, sin and cos are short series
 * in plain double arithmetic (no C library calls), so the bytes do not depend
 * on the host's libm.  The variate is formed in double,
 * narrowed to fp32, multiplied by the fp32 scale (and, for outlier channels,
 * by the fp32 channel multiplier), then rounded to bf16 with
 * round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one (seed, stream) pair; streams are independent sequences. */
uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN_GAMMA) ^ mix64(stream * 0xD1B54A32D192ED03ULL + 1ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t c) { return mix64(key + (c + 1ULL) * GOLDEN_GAMMA); }

/* Raw 64-bit draws for counters [c0, c0 + n). */
void synth_u64(uint64_t* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0) {
  const uint64_t key = synth_key(seed, stream);
  for (int64_t k = 0; k < n; ++k) dst[k] = draw(key, (uint64_t)(c0 + k));
}

/* Uniforms in [0, 1) with 53 random bits, counters [c0, c0 + n). */
void synth_uniform_f64(double* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0) {
  const uint64_t key = synth_key(seed, stream);
  for (int64_t k = 0; k < n; ++k) dst[k] = (double)(draw(key, (uint64_t)(c0 + k)) >> 11) * 0x1.0p-53;
}

/* Natural log of x > 0 (finite, normal): x = m 2^e with m in [sqrt(1/2), sqrt(2)),
 * log m = 2 atanh(s), s = (m - 1)/(m + 1), |s| <= 0.1716; the odd series to
 * s^11 leaves a relative error below 1e-11.  Plain arithmetic, so the values do
 * not depend on the C library. */
static inline double log_pos(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  b = (b & 0x000FFFFFFFFFFFFFULL) | 0x3FF0000000000000ULL;
  double m;
  memcpy(&m, &b, 8);
  if (m > 1.4142135623730951) {
    m *= 0.5;
    e += 1;
  }
  const double s = (m - 1.0) / (m + 1.0), s2 = s * s;
  const double p =
      s * (2.0 + s2 * (2.0 / 3 + s2 * (2.0 / 5 + s2 * (2.0 / 7 + s2 * (2.0 / 9 + s2 * (2.0 / 11))))));
  return p + (double)e * 0.69314718055994530942;
}

/* cos and sin of 2 pi u for u in [0, 1): quadrant q = round(4u), remainder
 * r = 2 pi (u - q/4) in [-pi/4, pi/4], Taylor series to r^14 / r^13. */
static inline void sincos_turn(double u, double* c, double* s) {
  const int q = (int)(u * 4.0 + 0.5);
  const double r = 6.283185307179586476925286766559 * (u - 0.25 * (double)q), r2 = r * r;
  const double sr = r * (1.0 - r2 / 6 * (1.0 - r2 / 20 * (1.0 - r2 / 42 * (1.0 - r2 / 72 * (1.0 - r2 / 110 *
                                                                                           (1.0 - r2 / 156))))));
  const double cr = 1.0 - r2 / 2 * (1.0 - r2 / 12 * (1.0 - r2 / 30 * (1.0 - r2 / 56 * (1.0 - r2 / 90 *
                                                                                        (1.0 - r2 / 132)))));
  switch (q & 3) {
    case 0: *c = cr; *s = sr; break;
    case 1: *c = -sr; *s = cr; break;
    case 2: *c = -cr; *s = -sr; break;
    default: *c = sr; *s = -cr; break;
  }
}

/* Both normals of pair p (counters 2p and 2p+1), in double. */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  const uint64_t b = draw(key, p);
  const double u1 = ((double)(b >> 40) + 0.5) * 0x1.0p-24;
  const double u2 = ((double)(b & 0xFFFFFFULL) + 0.5) * 0x1.0p-24;
  const double r = sqrt(-2.0 * log_pos(u1));
  double c, sn;
  sincos_turn(u2, &c, &sn);
  *z0 = r * c;
  *z1 = r * sn;
}

/* Standard normal for counter c, in double. */
static inline double normal_at(uint64_t key, uint64_t c) {
  double z0, z1;
  normal_pair(key, c >> 1, &z0, &z1);
  return (c & 1ULL) ? z1 : z0;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp32 values scale * N(0,1) for counters [c0, c0 + n). */
void synth_normal_f32(float* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0, float scale) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) dst[k] = (float)normal_at(key, (uint64_t)(c0 + k)) * scale;
}

/*
 * bf16 rows: dst[r][d] for rows r = 0..rows-1 (row index row0 + r in the
 * stream) and d = 0..D-1 uses counter (row0 + r) * D + d, so a row's values do
 * not depend on how many rows are drawn.  chan_mult (nullable, [D]) multiplies
 * channel d after the scale.
 */
void synth_rows_bf16(uint16_t* dst, int64_t rows, int64_t D, uint64_t seed, uint64_t stream, int64_t row0,
                     float scale, const float* chan_mult) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint64_t base = (uint64_t)(row0 + r) * (uint64_t)D;
    uint16_t* o = dst + r * D;
    int64_t d = 0;
    if (base & 1ULL) { /* odd start: first value is the sine branch of its pair */
      float v = (float)normal_at(key, base) * scale;
      if (chan_mult) v = v * chan_mult[0];
      o[0] = f32_to_bf16_rne(v);
      d = 1;
    }
    for (; d + 1 < D; d += 2) {
      double z0, z1;
      normal_pair(key, (base + (uint64_t)d) >> 1, &z0, &z1);
      float v0 = (float)z0 * scale, v1 = (float)z1 * scale;
      if (chan_mult) { v0 = v0 * chan_mult[d]; v1 = v1 * chan_mult[d + 1]; }
      o[d] = f32_to_bf16_rne(v0);
      o[d + 1] = f32_to_bf16_rne(v1);
    }
    if (d < D) {
      float v = (float)normal_at(key, base + (uint64_t)d) * scale;
      if (chan_mult) v = v * chan_mult[d];
      o[d] = f32_to_bf16_rne(v);
    }
  }
}
