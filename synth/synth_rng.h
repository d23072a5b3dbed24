/*
 * synth_rng.h - seeded, counter-based generator for synthetic inputs.
 *
 * This header is the single definition of every random input used by the
 * tests and the benchmark: weights, cached K/V values and token ids.  It is
 * compiled into a host library (synth_host.c, used by the CPU reference) and
 * into a GPU fill library (synth_gpu.hip, used to populate device memory).
 * Both produce bit-identical values because every step below is integer
 * arithmetic followed by one correctly rounded fp32 multiply.
 *
 * It contains none of the decode arithmetic; it only makes inputs.
 *
 * Generator
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014; the finaliser constants are the ones Vigna
 *     publishes with xoshiro).  The c-th output of a SplitMix64 stream with
 *     state `key` is mix(key + (c + 1) * GAMMA), so any element can be drawn
 *     independently of the others (counter-based use).
 *   - One stream per tensor: key = mix(mix(seed) ^ stream * 0xD1B54A32D192ED03).
 *   - Approximate standard normal: sum of twelve independent uniforms minus six
 *     (the classical Irwin-Hall approximation, variance exactly 1 in the limit
 *     of continuous uniforms).  The twelve uniforms are the 16-bit fields of
 *     the outputs at counters 3i, 3i+1 and 3i+2.  With u_j in [0, 65535] the
 *     centred integer numerator is N = sum(u_j) - 393210, and the deviate is
 *     N / 65536 (exact in fp32 since |N| < 2^19).  A value of scale s is
 *     N * (s * 2^-16), one fp32 multiply, then rounded to bf16
 *     (round-to-nearest-even) where a bf16 tensor is wanted.
 *   - RMSNorm gains: 1 + 0.25 * deviate (synth_gain_bf16), so that every gain differs
 *     from one and a kernel that drops the gain multiply, or reads another layer's
 *     gains, gives different results.
 */
#ifndef SYNTH_RNG_H
#define SYNTH_RNG_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN static inline __host__ __device__
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* c-th output (c = 0, 1, ...) of the SplitMix64 stream whose state is key. */
SYNTH_FN uint64_t synth_draw(uint64_t key, uint64_t c) {
  return synth_mix64(key + (c + 1ull) * SYNTH_GAMMA);
}

/* Per-tensor stream key. */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(synth_mix64(seed) ^ (stream * 0xD1B54A32D192ED03ull));
}

/* Centred integer numerator of the i-th approximate normal deviate. */
SYNTH_FN int32_t synth_normal_num(uint64_t key, uint64_t i) {
  int32_t s = 0;
  for (int j = 0; j < 3; ++j) {
    uint64_t w = synth_draw(key, 3ull * i + (uint64_t)j);
    s += (int32_t)(w & 0xffffu) + (int32_t)((w >> 16) & 0xffffu) +
         (int32_t)((w >> 32) & 0xffffu) + (int32_t)((w >> 48) & 0xffffu);
  }
  return s - 393210;
}

/* fp32 multiplier for deviates of standard deviation `scale`. */
SYNTH_FN float synth_scale_factor(float scale) { return scale * (1.0f / 65536.0f); }

/* i-th deviate of standard deviation scale (one rounded fp32 multiply). */
SYNTH_FN float synth_normal_f32(uint64_t key, uint64_t i, float factor) {
  return (float)synth_normal_num(key, i) * factor;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* i-th RMSNorm gain: bf16(1 + 0.25 * deviate).  The deviate's numerator N is an
   integer with |N| < 2^19, so N * 2^-18 and 1 + N * 2^-18 are exact in fp32 (at most
   21 significant bits): the value is the same whether or not a compiler fuses the
   multiply and the add, and the one rounding is the bf16 conversion. */
SYNTH_FN uint16_t synth_gain_bf16(uint64_t key, uint64_t i) {
  return synth_f32_to_bf16(1.0f + (float)synth_normal_num(key, i) * (1.0f / 262144.0f));
}

/* i-th uniform integer in [0, n). */
SYNTH_FN uint32_t synth_uniform_int(uint64_t key, uint64_t i, uint32_t n) {
  return (uint32_t)(((synth_draw(key, i) >> 32) * (uint64_t)n) >> 32);
}

#endif /* SYNTH_RNG_H */
