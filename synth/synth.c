/* Seeded synthetic inputs shared by the oracle tests and the GPU path.
 *
 * This module only draws numbers; it holds none of the decode step's
 * arithmetic.  Everything is counter-based so any element can be produced
 * independently (and in parallel):
 *
 *   splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014): the k-th output for seed s is
 *   mix(s + (k+1) * 0x9E3779B97F4A7C15) with the published finaliser
 *   mix(z) = z ^ (z >> 31) after two xor-shift-multiply rounds.
 *
 *   A tensor's own seed is output number `stream` of the base seed, so tensors
 *   drawn from different streams do not overlap.
 *
 *   Normal variates use the Box-Muller transform (cosine branch) on two
 *   consecutive outputs 2i and 2i+1: u1 in (0,1], u2 in [0,1).
 *
 *   bfloat16 storage: the float32 value rounded to nearest, ties to even, on
 *   the upper 16 bits.
 */
#include <math.h>
#include <stdint.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* k-th output (k >= 0) of splitmix64 started from `seed`. */
uint64_t synth_splitmix64(uint64_t seed, uint64_t k) {
  return sm_mix(seed + (k + 1) * 0x9E3779B97F4A7C15ULL);
}

uint64_t synth_stream_seed(uint64_t seed, uint64_t stream) {
  return synth_splitmix64(seed, stream);
}

static inline double sm_normal(uint64_t s, int64_t i) {
  const uint64_t a = synth_splitmix64(s, 2 * (uint64_t)i);
  const uint64_t b = synth_splitmix64(s, 2 * (uint64_t)i + 1);
  const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

static inline uint16_t sm_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  if ((v.u & 0x7F800000u) == 0x7F800000u && (v.u & 0x007FFFFFu)) return (uint16_t)((v.u >> 16) | 0x40u);
  const uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

/* out[i] = mean + scale * N(0,1), i in [0, n). */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double mean,
                      double scale, float* out) {
  const uint64_t s = synth_stream_seed(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + scale * sm_normal(s, i));
}

/* As synth_normal_f32, stored as bfloat16 bits (float32 value, then RNE). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double mean,
                       double scale, uint16_t* out) {
  const uint64_t s = synth_stream_seed(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sm_f32_to_bf16((float)(mean + scale * sm_normal(s, i)));
}

/* out[i] uniform in [lo, hi) from the top 32 bits of output i (multiply-shift). */
void synth_uniform_i32(uint64_t seed, uint64_t stream, int64_t n, int32_t lo,
                       int32_t hi, int32_t* out) {
  const uint64_t s = synth_stream_seed(seed, stream);
  const uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t a = synth_splitmix64(s, (uint64_t)i);
    out[i] = (int32_t)((int64_t)lo + (int64_t)(((a >> 32) * span) >> 32));
  }
}
