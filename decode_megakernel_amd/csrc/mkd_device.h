// mkd_device.h - device primitives for the decode megakernel on gfx950 (CDNA4).
//
// Counter protocol ("Inside the megakernel serving engine for North Mini Code",
// section "Barriers": a waiter spins until the counter reaches its target and then
// fences; an arriver fences its results and then atomically adds one).  On MI355X
// the eight XCDs have private L2 caches that are not coherent with each other, so
// both sides use agent-scope ordering: the arriver makes every wave's stores
// complete, then one lane issues an agent-scope release fence (L2 write-back) and
// a relaxed agent-scope atomic add; the waiter polls with relaxed agent-scope loads
// (which bypass the non-coherent cache levels), then issues an agent-scope acquire
// fence (cache invalidate) before the workgroup reads the producer's data.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mkd_common.h"

namespace mkd {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kWreg = 16;  // 16-byte weight chunks held in registers per lane

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ loads
// Streaming (non-temporal) 16-byte load for weights and cached K/V: read once per
// step, so they should not displace activations from the caches.
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld_stream8(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// sum_k w[k] * x[k] over 8 bf16 weights and 8 fp32 activations.
__device__ __forceinline__ float dot8(const u32x4 w, const float4 a, const float4 b) {
  float s = bf_lo(w.x) * a.x;
  s = fmaf(bf_hi(w.x), a.y, s);
  s = fmaf(bf_lo(w.y), a.z, s);
  s = fmaf(bf_hi(w.y), a.w, s);
  s = fmaf(bf_lo(w.z), b.x, s);
  s = fmaf(bf_hi(w.z), b.y, s);
  s = fmaf(bf_lo(w.w), b.z, s);
  s = fmaf(bf_hi(w.w), b.w, s);
  return s;
}

// ------------------------------------------------------------------ wave reductions
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ------------------------------------------------------------------ counters
__device__ __forceinline__ uint32_t ctr_load(const uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_add(uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
// Wait until this wave's own outstanding vector memory operations (its stores in
// particular) have completed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t* gctr(const Params& p, int which) {
  return p.counters + p.ctr.global_base + which;
}
__device__ __forceinline__ bool aborted(const Params& p) { return ctr_load(gctr(p, G_ABORT)) != 0; }

// Record the first device-side error and stop every workgroup.
__device__ inline void report_error(const Params& p, uint32_t code, int32_t task, int32_t ctr,
                                    uint32_t seen, uint32_t want) {
  if (atomicCAS(gctr(p, G_ERR_CODE), 0u, code) == 0u) {
    *gctr(p, G_ERR_TASK) = (uint32_t)task;
    *gctr(p, G_ERR_CTR) = (uint32_t)ctr;
    *gctr(p, G_ERR_SEEN) = seen;
    *gctr(p, G_ERR_WANT) = want;
  }
  if (code == 1u) {
    fence_release_agent();
    ctr_add(gctr(p, G_ABORT), 1u);
  }
}

}  // namespace mkd
