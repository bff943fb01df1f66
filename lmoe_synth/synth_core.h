/* Seeded synthetic inputs for the Stable LatentMoE layer: one counter-based
 * generator, written once and compiled for the host (gcc) and for the device
 * (hipcc).  It holds none of the layer's arithmetic; it only turns
 * (seed, tensor id, element index) into a number.
 *
 * Definition (every element is a pure function of its coordinates):
 *   key      = splitmix64_mix(seed * 65536 + tensor_id)
 *   h1, h2   = outputs 2i and 2i+1 of the SplitMix64 stream started at key,
 *              i.e. splitmix64_mix(key + (2i+1)*G) and splitmix64_mix(key + (2i+2)*G)
 *              with G = 0x9E3779B97F4A7C15 (Steele, Lea & Flood, "Fast
 *              splittable pseudorandom number generators", OOPSLA 2014; the
 *              mixing function is the one used by SplitMix64 / SplittableRandom).
 *   u1       = ((h1 >> 11) + 1) * 2^-53          in (0, 1]
 *   u2       = (h2 >> 11) * 2^-53                in [0, 1)
 *   normal   = sqrt(-2 ln u1) * cos(2 pi u2)     (Box & Muller, 1958), fp64
 *   uniform  = lo + (hi - lo) * u2               fp64
 *   value    = normal * scale * (row multiplier), fp64, then rounded to fp32 (RNE),
 *              then, for bf16 storage, fp32 -> bf16 (RNE).
 *
 * ln and cos come from the platform's fp64 libm (glibc on the host, the ROCm
 * device library on the GPU).  Both are faithfully rounded; a one-ulp fp64
 * difference changes a stored bf16 value only when the fp64 value sits within
 * one ulp of a bf16 rounding midpoint (odds ~2^-44 per element).
 */
#ifndef LMOE_SYNTH_CORE_H
#define LMOE_SYNTH_CORE_H

#include <stdint.h>
#include <math.h>
#include <string.h>

#if defined(__HIPCC__)
#define LMOE_SYNTH_FN __host__ __device__ static inline
#else
#define LMOE_SYNTH_FN static inline
#endif

#define LMOE_SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

LMOE_SYNTH_FN uint64_t lmoe_synth_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

LMOE_SYNTH_FN uint64_t lmoe_synth_key(uint64_t seed, uint32_t tensor_id) {
  return lmoe_synth_mix(seed * 65536ULL + (uint64_t)tensor_id);
}

/* u1 in (0,1], u2 in [0,1) for element i of the stream `key`. */
LMOE_SYNTH_FN void lmoe_synth_uniform_pair(uint64_t key, uint64_t i, double* u1, double* u2) {
  uint64_t h1 = lmoe_synth_mix(key + (2 * i + 1) * LMOE_SYNTH_GAMMA);
  uint64_t h2 = lmoe_synth_mix(key + (2 * i + 2) * LMOE_SYNTH_GAMMA);
  const double two_m53 = 1.1102230246251565e-16; /* 2^-53, exact */
  *u1 = (double)((h1 >> 11) + 1) * two_m53;
  *u2 = (double)(h2 >> 11) * two_m53;
}

LMOE_SYNTH_FN double lmoe_synth_normal(uint64_t key, uint64_t i) {
  double u1, u2;
  lmoe_synth_uniform_pair(key, i, &u1, &u2);
  const double two_pi = 6.283185307179586;
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

LMOE_SYNTH_FN double lmoe_synth_uniform(uint64_t key, uint64_t i, double lo, double hi) {
  double u1, u2;
  lmoe_synth_uniform_pair(key, i, &u1, &u2);
  return lo + (hi - lo) * u2;
}

/* fp32 -> bf16 bits, round to nearest even (values here are finite). */
LMOE_SYNTH_FN uint16_t lmoe_synth_f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb;
  return (uint16_t)(b >> 16);
}

/* Element value before storage rounding: normal * scale, times row_mult for
 * the first `rows_mult` rows of length `row_len` (used to skew router rows). */
LMOE_SYNTH_FN double lmoe_synth_normal_value(uint64_t key, uint64_t i, double scale,
                                             int64_t row_len, int64_t rows_mult, double row_mult) {
  double v = lmoe_synth_normal(key, i) * scale;
  if (rows_mult > 0 && row_len > 0 && (int64_t)(i / (uint64_t)row_len) < rows_mult) v = v * row_mult;
  return v;
}

#endif
