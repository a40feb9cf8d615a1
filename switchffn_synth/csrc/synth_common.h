/*
 * Counter-based synthetic input generator shared by the test/bench harness.
 *
 * This header holds no step of the SwitchFFN method: it only defines how the
 * seeded synthetic inputs (token states and weights) are produced, so that the
 * host (C, for the CPU oracle) and the device (HIP, for filling large weight
 * tensors in place) produce the same bytes for every element.
 *
 * Definition (random access, element i of stream s under seed S):
 *   key    = mix64(S * GOLDEN + mix64(s + GOLDEN))
 *   w_j    = mix64(key + (3*i + j + 1) * GOLDEN),  j = 0, 1, 2
 *   U      = sum of the twelve 16-bit fields of w_0, w_1, w_2   (0 .. 786420)
 *   z      = (float)(U - 393210) * 2^-16      (exact in fp32; mean 0, var ~1)
 *   value  = z * sigma                         (one IEEE fp32 multiply, RNE)
 *   bf16   = round-to-nearest-even of value to bfloat16 (when requested)
 * mix64 is the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) and GOLDEN its
 * increment. The sum of twelve uniforms is the classical Irwin-Hall
 * approximation of a standard normal (bounded at +-6 sigma).
 */
#ifndef SWITCHFFN_SYNTH_COMMON_H
#define SWITCHFFN_SYNTH_COMMON_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GOLDEN 0x9e3779b97f4a7c15ULL

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(seed * SYNTH_GOLDEN + synth_mix64(stream + SYNTH_GOLDEN));
}

SYNTH_FN uint32_t synth_fields16(uint64_t w) {
  return (uint32_t)(w & 0xffffu) + (uint32_t)((w >> 16) & 0xffffu) +
         (uint32_t)((w >> 32) & 0xffffu) + (uint32_t)(w >> 48);
}

/* Irwin-Hall(12) value for element index i, scaled by sigma, as fp32. */
SYNTH_FN float synth_value(uint64_t key, uint64_t i, float sigma) {
  uint64_t c = key + (3u * i + 1u) * SYNTH_GOLDEN;
  uint32_t u = synth_fields16(synth_mix64(c)) +
               synth_fields16(synth_mix64(c + SYNTH_GOLDEN)) +
               synth_fields16(synth_mix64(c + 2u * SYNTH_GOLDEN));
  float z = (float)((int32_t)u - 393210) * 0.0000152587890625f; /* 2^-16 */
  return z * sigma;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs only). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif
