// mkd_device.h - device primitives for the decode megakernel on gfx950 (CDNA4).
//
// Dependency protocol ("Inside the megakernel serving engine for North Mini Code",
// section "Barriers": a waiter spins until its dependency is met and then reads the
// producer's data).  On MI355X the eight XCDs have private L2 caches that are not
// coherent with each other.  Data that crosses workgroups travels as tagged 64-bit words
// (value and a step/layer tag, one agent-scope store, written through to the coherent
// level): the consumer polls the words themselves with agent-scope loads, which bypass
// the non-coherent levels, so no fence or atomic sits on the critical path.  Counters
// (relaxed agent-scope atomics) remain for the claim queues and the abort / error block;
// the one plain-load consumer of data written during the step (the new K/V slot of the
// paged pool) waits on tagged flags and then issues an agent-scope acquire.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mkd_common.h"

namespace mkd {

// Address spaces: global memory (1) and LDS (3).  Every pointer the kernels use
// carries its address space so that the compiler emits global_* and ds_*
// instructions: a generic (flat) access would count against both the vector-memory
// and the LDS wait counters, making every LDS access and barrier wait for all weight
// loads in flight.
#define GAS __attribute__((address_space(1)))
#define LAS __attribute__((address_space(3)))
// Read-only inputs (task lists, token ids, lengths, page tables) are read through the
// constant address space, so wave-uniform reads become scalar loads.
#define CAS __attribute__((address_space(4)))

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ loads
// Streaming (non-temporal) 16-byte load for weights and cached K/V: read once per
// step, so they should not displace activations from the caches.
__device__ __forceinline__ u32x4 ld_stream16(const GAS void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const GAS u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld_stream8(const GAS void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const GAS u32x2*>(p));
}
// Streaming 16-byte load of each lane straight into LDS (global_load_lds_dwordx4, no
// registers involved): lane i's bytes land at lds + 16 * i, lds being wave-uniform.  The
// load counts on the vector-memory counter like any other; the LDS bytes may be read once
// the issuing wave has waited for it (only the issuing wave reads them here).
__device__ __forceinline__ void dma16(const GAS void* p, LAS void* lds) {
  __builtin_amdgcn_global_load_lds(p, lds, 16, 0, 2 /* nt */);
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
// The same for finite values, by CDNA4's packed conversion (one instruction).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// sum_k w[k] * x[k] over 8 bf16 weights and 8 fp32 activations.
__device__ __forceinline__ float dot8(const u32x4 w, const f32x4 a, const f32x4 b) {
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
// Cross-lane sums and maxima with DPP row rotations (every lane of a 16-lane row ends with
// the row's result after four rotate-and-combine steps) and readlane for combining rows:
// no LDS round trip per step, unlike a shuffle through ds_bpermute.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
// DPP row_ror:n = 0x120 + n
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x122>(v);
  v += dpp_f<0x121>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0x128>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x122>(v));
  v = fmaxf(v, dpp_f<0x121>(v));
  return v;
}
__device__ __forceinline__ int row16_min(int v) {
  v = min(v, dpp_i<0x128>(v));
  v = min(v, dpp_i<0x124>(v));
  v = min(v, dpp_i<0x122>(v));
  v = min(v, dpp_i<0x121>(v));
  return v;
}
// Maximum / sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48),
// returned to every lane, by CDNA4's lane swaps between register halves and row pairs (two
// VALU instructions each, no LDS round trip).  Every lane adds the same two partial sums,
// so the four lanes of a column get the same value.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Sum over aligned groups of WIDTH lanes, returned to every lane of the group.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (WIDTH == 64) {
    const float r = row16_sum(v);
    return (lane_f(r, 0) + lane_f(r, 16)) + (lane_f(r, 32) + lane_f(r, 48));
  } else if constexpr (WIDTH == 32) {
    const float r = row16_sum(v);
    const float lo = lane_f(r, 0) + lane_f(r, 16), hi = lane_f(r, 32) + lane_f(r, 48);
    return (threadIdx.x & 32) ? hi : lo;
  } else if constexpr (WIDTH == 16) {
    return row16_sum(v);
  } else {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
  }
}
__device__ __forceinline__ float wave_max(float v) {
  const float r = row16_max(v);
  return fmaxf(fmaxf(lane_f(r, 0), lane_f(r, 16)), fmaxf(lane_f(r, 32), lane_f(r, 48)));
}
__device__ __forceinline__ int wave_min_i(int v) {
  const int r = row16_min(v);
  return min(min(__builtin_amdgcn_readlane(r, 0), __builtin_amdgcn_readlane(r, 16)),
             min(__builtin_amdgcn_readlane(r, 32), __builtin_amdgcn_readlane(r, 48)));
}
// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ------------------------------------------------------------------ counters
__device__ __forceinline__ uint32_t ctr_load(const GAS uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_add(GAS uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_cas(GAS uint32_t* c, uint32_t expect, uint32_t v) {
  __hip_atomic_compare_exchange_strong(c, &expect, v, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return expect;
}
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
// Wait until this wave's own outstanding vector memory operations (its stores in
// particular) have completed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stores of data that other workgroups read during the same step.  An agent-scope
// atomic store is written through the XCD's L2 to the device-coherent level (it must be
// visible to agent-scope loads on every XCD without any fence after it), so a producer
// publishes such data by waiting for its own stores to complete and then adding to the
// counter: no agent-scope release fence, whose L2 write-back of every dirty line costs
// microseconds.  Consumers still acquire (invalidate) before reading with plain loads.
// Outputs the host reads (logits, debug buffers) use them too, so that they are in memory
// whatever release the end of the dispatch performs.
__device__ __forceinline__ void st_pub(GAS float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_pub(GAS int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_pub(GAS uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_pub4(GAS float* p, f32x4 v) {
  GAS uint64_t* q = reinterpret_cast<GAS uint64_t*>(p);
  __hip_atomic_store(q, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged words.  Data that one workgroup produces and another consumes during the step
// travels as 64-bit words: the fp32 payload in the low half and the step's epoch in the
// high half, written with one agent-scope store (single-copy atomic, written through to
// the device-coherent level).  A consumer reads the words with agent-scope loads and
// retries those whose tag is not yet this step's: the data is its own ready flag, so an
// edge costs the producer's store and the consumer's load, where a counter costs the
// store, the wait for its completion, the atomic add, the counter poll, the acquire and
// then the load.  The tag names the step and the layer, (epoch << 8) | layer, because
// some buffers (the attention partials) are reused by every layer of a step; words left
// from earlier layers or steps carry other tags.
__device__ __forceinline__ uint32_t layer_tag(uint32_t epoch, int layer) { return (epoch << 8) | (uint32_t)layer; }
__device__ __forceinline__ uint64_t tag_word(float v, uint32_t ep) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)ep << 32);
}
__device__ __forceinline__ void st_tag(GAS uint64_t* p, float v, uint32_t ep) {
  __hip_atomic_store(p, tag_word(v, ep), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const GAS uint64_t* p) {
  return __hip_atomic_load(const_cast<GAS uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t ep) { return (uint32_t)(w >> 32) == ep; }
__device__ __forceinline__ float tag_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Device view of the kernel parameters: the same fields, with address-space
// qualified pointers.
struct DParams {
  int32_t n_layers, hidden, n_q, n_kv, head_dim, n_experts, top_k, inter, vocab, page;
  float rms_eps;
  int32_t batch, max_batch, max_pages, n_pages;
  PlanShape shape;
  CounterLayout ctr;
  const GAS uint16_t* embed;
  const GAS uint16_t* norm;
  const GAS uint16_t* w_qkv;
  const GAS uint16_t* w_o;
  const GAS uint16_t* w_router;
  const GAS uint16_t* w_gate_up;
  const GAS uint16_t* w_down;
  const CAS int32_t* tokens;
  const CAS int32_t* seq_lens;
  const CAS int32_t* page_table;
  GAS uint16_t* kv_pool;
  GAS float* logits;
  GAS uint64_t* h;
  GAS uint64_t* ss;
  GAS uint64_t* q;
  GAS uint64_t* kvflag;
  GAS uint64_t* attn_part;
  GAS uint64_t* attn_o;
  GAS uint64_t* router;
  GAS uint64_t* route_tbl;
  GAS int32_t* topk_ids;
  GAS float* topk_w;
  GAS uint64_t* moe_act;
  GAS uint64_t* moe_part;
  const CAS double* inv_freq;
  GAS uint64_t* rope;
  GAS uint32_t* counters;
  const CAS int32_t* tasks;
  const CAS int32_t* cu_offsets;
  int32_t max_attn_items;
  int32_t spin_limit;
  uint32_t epoch;
  GAS uint64_t* trace;
  int32_t trace_cap;
  int32_t attn_window, full_every;
};

template <typename T>
__device__ __forceinline__ GAS T* gas(T* p) {
  return (GAS T*)p;
}
template <typename T>
__device__ __forceinline__ const CAS T* cas(const T* p) {
  return (const CAS T*)p;
}

// Kernel arguments read through the constant address space (scalar loads).
typedef const __attribute__((address_space(4))) Params KParams;

__device__ __forceinline__ DParams device_view(KParams& p) {
  DParams d;
  d.n_layers = p.n_layers; d.hidden = p.hidden; d.n_q = p.n_q; d.n_kv = p.n_kv; d.head_dim = p.head_dim;
  d.n_experts = p.n_experts; d.top_k = p.top_k; d.inter = p.inter; d.vocab = p.vocab; d.page = p.page;
  d.rms_eps = p.rms_eps;
  d.batch = p.batch; d.max_batch = p.max_batch; d.max_pages = p.max_pages; d.n_pages = p.n_pages;
  d.shape.n_rt = p.shape.n_rt; d.shape.rt_rows = p.shape.rt_rows;
  d.shape.up_rows = p.shape.up_rows; d.shape.n_up_tiles = p.shape.n_up_tiles;
  d.shape.pages_per_item = p.shape.pages_per_item; d.shape.qkv_rows = p.shape.qkv_rows; d.shape.qkv_tph = p.shape.qkv_tph;
  d.shape.router_rows = p.shape.router_rows; d.shape.lm_rows = p.shape.lm_rows;
  d.shape.down_rows = p.shape.down_rows; d.shape.n_down_chunks = p.shape.n_down_chunks;
  d.ctr.per_layer = p.ctr.per_layer; d.ctr.attn_claim = p.ctr.attn_claim; d.ctr.up_claim = p.ctr.up_claim;
  d.ctr.down_claim = p.ctr.down_claim;
  d.ctr.global_base = p.ctr.global_base;
  d.ctr.total = p.ctr.total;
  d.embed = gas(p.embed); d.norm = gas(p.norm); d.w_qkv = gas(p.w_qkv); d.w_o = gas(p.w_o);
  d.w_router = gas(p.w_router); d.w_gate_up = gas(p.w_gate_up); d.w_down = gas(p.w_down);
  d.tokens = cas(p.tokens); d.seq_lens = cas(p.seq_lens); d.page_table = cas(p.page_table);
  d.kv_pool = gas(p.kv_pool); d.logits = gas(p.logits);
  d.h = gas(p.h); d.ss = gas(p.ss); d.q = gas(p.q); d.kvflag = gas(p.kvflag); d.attn_part = gas(p.attn_part); d.attn_o = gas(p.attn_o);
  d.router = gas(p.router); d.route_tbl = gas(p.route_tbl); d.topk_ids = gas(p.topk_ids); d.topk_w = gas(p.topk_w);
  d.moe_act = gas(p.moe_act); d.moe_part = gas(p.moe_part); d.inv_freq = cas(p.inv_freq);
  d.rope = gas(p.rope);
  d.counters = gas(p.counters); d.tasks = cas(p.tasks); d.cu_offsets = cas(p.cu_offsets);
  d.max_attn_items = p.max_attn_items; d.spin_limit = p.spin_limit; d.epoch = p.epoch;
  d.trace = gas(p.trace); d.trace_cap = p.trace_cap;
  d.attn_window = p.attn_window; d.full_every = p.full_every;
  return d;
}

__device__ __forceinline__ GAS uint32_t* gctr(const DParams& p, int which) {
  return p.counters + p.ctr.global_base + which;
}
__device__ __forceinline__ bool aborted(const DParams& p) { return ctr_load(gctr(p, G_ABORT)) != 0; }

// Record the first device-side error and stop every workgroup.
__device__ inline void report_error(const DParams& p, uint32_t code, int32_t task, int32_t ctr,
                                    uint32_t seen, uint32_t want) {
  if (ctr_cas(gctr(p, G_ERR_CODE), 0u, code) == 0u) {
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
