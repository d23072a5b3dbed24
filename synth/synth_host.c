/*
 * synth_host.c - CPU fill functions for the seeded synthetic inputs.
 * Definitions of the generator are in synth_rng.h; the GPU fill library
 * (synth_gpu.hip) produces the same values element for element.
 */
#include <stdint.h>
#include "synth_rng.h"

/* dst[j] = bf16(normal(seed, stream, offset + j) * scale), j in [0, n). */
void synth_host_normal_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                            float scale, uint64_t offset) {
  const uint64_t key = synth_key(seed, stream);
  const float factor = synth_scale_factor(scale);
#pragma omp parallel for schedule(static)
  for (long long j = 0; j < (long long)n; ++j)
    dst[j] = synth_f32_to_bf16(synth_normal_f32(key, offset + (uint64_t)j, factor));
}

/* dst[j] = normal(seed, stream, offset + j) * scale in fp32. */
void synth_host_normal_f32(float* dst, uint64_t n, uint64_t seed, uint64_t stream,
                           float scale, uint64_t offset) {
  const uint64_t key = synth_key(seed, stream);
  const float factor = synth_scale_factor(scale);
#pragma omp parallel for schedule(static)
  for (long long j = 0; j < (long long)n; ++j)
    dst[j] = synth_normal_f32(key, offset + (uint64_t)j, factor);
}

/* dst[j] = bf16 RMSNorm gain at counter offset + j (synth_gain_bf16). */
void synth_host_gain_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t stream, uint64_t offset) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (long long j = 0; j < (long long)n; ++j) dst[j] = synth_gain_bf16(key, offset + (uint64_t)j);
}

/* dst[j] = uniform integer in [0, range) at counter offset + j. */
void synth_host_uniform_int(int32_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                            uint32_t range, uint64_t offset) {
  const uint64_t key = synth_key(seed, stream);
  for (uint64_t j = 0; j < n; ++j) dst[j] = (int32_t)synth_uniform_int(key, offset + j, range);
}
