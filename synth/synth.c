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
 * counter 2p+1 the sine branch of pair p.  The variate is formed in double,
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

/* Both normals of pair p (counters 2p and 2p+1), in double. */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  const uint64_t b = draw(key, p);
  const double u1 = ((double)(b >> 40) + 0.5) * 0x1.0p-24;
  const double u2 = ((double)(b & 0xFFFFFFULL) + 0.5) * 0x1.0p-24;
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(th);
  *z1 = r * sin(th);
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
