/*
 * Seeded, counter-based synthetic input generator (host side).
 *
 * This module only draws numbers; it holds none of the Switch layer's
 * arithmetic.  Both the HIP library's tests/benchmark and the CPU oracle take
 * their inputs from here, so they see identical values.
 *
 * Definition (every element is independent, so any slice can be regenerated
 * on its own, e.g. one expert's weights of a 100 GB weight bank):
 *
 *   stream      = mix64(seed * 2^8 + tensor_id + 1)
 *   draw(n)     = mix64(stream + (n + 1) * GAMMA)
 *                 i.e. the n-th output of SplitMix64 seeded with `stream`
 *                 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *                 generators", OOPSLA 2014; finalizer constants from there).
 *   element i, attempt a (0 <= a < 64), lane j in {0,1}:
 *                 n = (i * 64 + a) * 2 + j
 *   uniform     u_j = (draw(n) >> 11) * 2^-52 - 1          in [-1, 1), exact
 *   normal      Marsaglia's polar method: s = u0^2 + u1^2; reject s >= 1 or
 *               s == 0; z = u0 * sqrt(-2 ln(s) / s)
 *   truncation  (truncated tensors) also reject |z| > 2
 *   value       (float)(z * std), and for bf16 tensors the round-to-nearest-
 *               even bf16 of that float
 *   If all 64 attempts are rejected (probability about 0.25^64 per element)
 *   the element is 0.
 *
 * ln() is evaluated here with +, -, *, / only (exponent split plus the atanh
 * series), so that a GPU implementation of the same definition produces the
 * same bits; the file is compiled with floating-point contraction disabled.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double u64_as_f64(uint64_t b) { double d; memcpy(&d, &b, 8); return d; }
static inline uint64_t f64_as_u64(double d) { uint64_t b; memcpy(&b, &d, 8); return b; }

/* natural log of a positive normal double using only IEEE basic operations */
static double synth_ln(double s) {
  uint64_t b = f64_as_u64(s);
  int e = (int)((b >> 52) & 0x7ff) - 1023;
  double m = u64_as_f64((b & 0x000FFFFFFFFFFFFFULL) | 0x3FF0000000000000ULL); /* [1,2) */
  if (m > 1.4142135623730951) { m = m * 0.5; e += 1; }
  double t = (m - 1.0) / (m + 1.0);
  double t2 = t * t;
  /* atanh series: ln m = 2 t (1 + t2/3 + t2^2/5 + ... ) */
  double p = 1.0 / 25.0;
  p = p * t2 + 1.0 / 23.0;
  p = p * t2 + 1.0 / 21.0;
  p = p * t2 + 1.0 / 19.0;
  p = p * t2 + 1.0 / 17.0;
  p = p * t2 + 1.0 / 15.0;
  p = p * t2 + 1.0 / 13.0;
  p = p * t2 + 1.0 / 11.0;
  p = p * t2 + 1.0 / 9.0;
  p = p * t2 + 1.0 / 7.0;
  p = p * t2 + 1.0 / 5.0;
  p = p * t2 + 1.0 / 3.0;
  p = p * t2 + 1.0;
  return (double)e * 0.6931471805599453 + 2.0 * t * p;
}

static inline double synth_uniform(uint64_t stream, uint64_t n) {
  uint64_t r = mix64(stream + (n + 1ULL) * SYNTH_GAMMA);
  return (double)(r >> 11) * (1.0 / 4503599627370496.0) - 1.0;
}

double synth_normal(uint64_t seed, uint32_t tensor_id, int truncated, uint64_t index) {
  uint64_t stream = mix64(seed * 256ULL + (uint64_t)tensor_id + 1ULL);
  for (uint64_t a = 0; a < 64; ++a) {
    uint64_t n = (index * 64ULL + a) * 2ULL;
    double u0 = synth_uniform(stream, n);
    double u1 = synth_uniform(stream, n + 1ULL);
    double s = u0 * u0 + u1 * u1;
    if (s >= 1.0 || s == 0.0) continue;
    double z = u0 * sqrt(-2.0 * synth_ln(s) / s);
    if (truncated && (z > 2.0 || z < -2.0)) continue;
    return z;
  }
  return 0.0;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_fill_f32(uint64_t seed, uint32_t tensor_id, int truncated, double std,
                    uint64_t start, uint64_t count, float* out, int nthreads) {
  (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = (float)(synth_normal(seed, tensor_id, truncated, start + (uint64_t)j) * std);
}

void synth_fill_bf16(uint64_t seed, uint32_t tensor_id, int truncated, double std,
                     uint64_t start, uint64_t count, uint16_t* out, int nthreads) {
  (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t j = 0; j < (int64_t)count; ++j)
    out[j] = f32_to_bf16_rne((float)(synth_normal(seed, tensor_id, truncated, start + (uint64_t)j) * std));
}

/* used by the tests of this module only: the unrounded log */
double synth_ln_export(double s) { return synth_ln(s); }
