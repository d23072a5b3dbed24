/*
 * synth_gpu.hip - GPU fill kernels for the seeded synthetic inputs.
 * Same generator as synth_host.c (definitions in synth_rng.h), so a tensor
 * filled here equals, bit for bit, the one the CPU fill would produce.
 * This library only makes inputs; it is not part of the decode path.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth_rng.h"

__global__ void __launch_bounds__(256)
synth_normal_bf16_kernel(uint16_t* __restrict__ dst, uint64_t n, uint64_t key, float factor,
                         uint64_t offset) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = synth_f32_to_bf16(synth_normal_f32(key, offset + j, factor));
}

__global__ void __launch_bounds__(256)
synth_gain_bf16_kernel(uint16_t* __restrict__ dst, uint64_t n, uint64_t key, uint64_t offset) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = synth_gain_bf16(key, offset + j);
}

__global__ void __launch_bounds__(256)
synth_fill_u16_kernel(uint16_t* __restrict__ dst, uint64_t n, uint16_t value) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = value;
}

static unsigned synth_grid(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return (unsigned)g;
}

extern "C" {

/* Fill n bf16 elements of device memory dst with normal(seed, stream, offset+j)*scale.
   Returns a hipError_t code (0 on success).  Asynchronous on `stream_handle`. */
int synth_gpu_normal_bf16(void* dst, uint64_t n, uint64_t seed, uint64_t stream, float scale,
                          uint64_t offset, void* stream_handle) {
  if (n == 0) return 0;
  const uint64_t key = synth_key(seed, stream);
  hipLaunchKernelGGL(synth_normal_bf16_kernel, dim3(synth_grid(n)), dim3(256), 0,
                     (hipStream_t)stream_handle, (uint16_t*)dst, n, key,
                     synth_scale_factor(scale), offset);
  return (int)hipGetLastError();
}

/* Fill n bf16 RMSNorm gains (synth_gain_bf16) at counters offset .. offset+n-1. */
int synth_gpu_gain_bf16(void* dst, uint64_t n, uint64_t seed, uint64_t stream, uint64_t offset,
                        void* stream_handle) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(synth_gain_bf16_kernel, dim3(synth_grid(n)), dim3(256), 0,
                     (hipStream_t)stream_handle, (uint16_t*)dst, n, synth_key(seed, stream), offset);
  return (int)hipGetLastError();
}

/* Fill n 16-bit elements of device memory with a constant bit pattern. */
int synth_gpu_fill_u16(void* dst, uint64_t n, uint32_t value, void* stream_handle) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(synth_fill_u16_kernel, dim3(synth_grid(n)), dim3(256), 0,
                     (hipStream_t)stream_handle, (uint16_t*)dst, n, (uint16_t)value);
  return (int)hipGetLastError();
}

}  // extern "C"
