/*
 * Seeded synthetic inputs shared by the GPU path and the CPU oracle.
 *
 * This file holds no arithmetic of the tensor-parallel method: it only draws
 * numbers.  Each logical tensor is addressed by (seed, stream); element i is a
 * pure function of (seed, stream, i), so any slice can be drawn on its own and
 * the draw parallelises without changing a single bit.
 *
 * Generator: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * Splittable Pseudorandom Number Generators", OOPSLA 2014) applied to the
 * counter key + (i + 1) * golden_gamma, and the Box-Muller transform (Box and
 * Muller, 1958) on the two 32-bit halves of that 64-bit word.
 *
 * bf16 outputs are the float32 value rounded to nearest-even (bf16 keeps the
 * top 16 bits of the float32 pattern).
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN_GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL + 1));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN_GAMMA);
}

static inline float normal_at(uint64_t key, uint64_t i, double scale) {
  uint64_t z = word_at(key, i);
  double u1 = ((double)(z >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(z & 0xFFFFFFFFULL) + 0.5) * (1.0 / 4294967296.0);
  double r = sqrt(-2.0 * log(u1));
  return (float)(scale * r * cos(6.283185307179586476925 * u2));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t lsb = (v.u >> 16) & 1u;
  v.u += 0x7FFFu + lsb;
  return (uint16_t)(v.u >> 16);
}

/* out[i] = scale * N(0,1)_i for i in [first, first + n). */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t first, int64_t n,
                      double scale, float* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, (uint64_t)(first + i), scale);
}

/* Same draw as synth_normal_f32, rounded once to bf16 (returned as raw bits). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t first, int64_t n,
                       double scale, uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne(normal_at(key, (uint64_t)(first + i), scale));
}

/* Integers uniform on [lo, hi] as float32 (exact: |values| < 2^24). */
void synth_int_f32(uint64_t seed, uint64_t stream, int64_t first, int64_t n,
                   int32_t lo, int32_t hi, float* out) {
  const uint64_t key = stream_key(seed, stream);
  const uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)((int64_t)lo + (int64_t)(word_at(key, (uint64_t)(first + i)) % span));
}
