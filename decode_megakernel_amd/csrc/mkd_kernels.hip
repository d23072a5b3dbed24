// mkd_kernels.hip - the decode megakernel for gfx950: tile bodies of every opcode and
// the persistent task interpreter (plus the op-per-kernel ablation launcher).
//
// Method: "Inside the megakernel serving engine for North Mini Code" (Cohere).
//  - "What is a Megakernel?": one workgroup per compute unit, resident for the whole
//    step, walking a host-built task list in global memory; dependencies are counters
//    that producers increment and consumers spin on.
//  - "The threadblock shape": every opcode runs under one fixed shape with fixed
//    roles.  Here: 8 wave64s; wave 0 is the controller (counter polls, queue claims,
//    activation staging into LDS, epilogue stores, fences and arrives) and waves 1..7
//    are workers that only stream weights / K-V from HBM and compute.  On gfx9 the
//    vector-memory counter is in order and shared by loads, stores and atomics, so a
//    wave with weight loads in flight cannot get a quick answer from a poll, a small
//    load or a store; keeping every latency-critical access on a wave that never
//    streams weights is what lets the workers keep HBM busy while the controller
//    resolves dependencies.  Barriers only order LDS, so worker loads stay in flight
//    across them.
//  - "Tasks": the GEMM opcodes share one body (a bf16 GEMV tile held in worker
//    registers, fp32 accumulation, wave reductions); QKV applies RoPE in the
//    epilogue; attention is split over KV slices and combined; routing scores the
//    experts and picks the top-k per token; expert gate/up fuses SiLU-and-multiply;
//    MOE_COMBINE weights expert outputs by router scores.
//  - "Weight prefetch" (section "Where the speedup comes from", item 3): weights never
//    depend on this step's activations, so workers issue a task's weight loads before
//    its input counter is satisfied, and move on to the next task's weights while the
//    controller finishes the previous epilogue.
//  - "The task scheduler": attention and MoE stages are drained by claimer tasks that
//    atomically take the next item of a shared queue until it is empty; the controller
//    claims item j+1 while the workers compute item j.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mkd_common.h"
#include "mkd_device.h"

namespace mkd {

// ------------------------------------------------------------------ LDS layout
// One workgroup per CU is forced by the LDS footprint (> half of the 160 KB).
constexpr int kLdsXs = 0;            // 128 KB: activation staging, attention merge / combine
constexpr int kLdsXsBytes = 131072;
constexpr int kLdsRowsum = 131072;   // 8 KB: per-row results of a tile
constexpr int kLdsRoute = 139264;    // 8 KB: routing tables
constexpr int kLdsMisc = 147456;     // 1 KB: broadcasts, controller state, inverse RMS
constexpr int kLdsBytes = 148480;
constexpr int kAttnMaxChunks = 1536;  // attention chunks per (sequence, KV group) combined in LDS
constexpr int kMaxPagesPerWave = 2;   // attention pages each worker holds in registers
#ifndef MKD_RING
#define MKD_RING 5
#endif
constexpr int kRing = MKD_RING;       // 16-byte weight chunks in flight per worker lane
constexpr int kMaxSteps = 5;          // row steps per worker in one GEMV tile
constexpr int kMaxBatch = 16;

struct Smem {
  LAS float* xs;
  LAS float* rowsum;
  LAS int32_t* route;
  LAS int32_t* mi;  // misc ints
  LAS float* mf;    // misc floats (inverse RMS per token)
  __device__ explicit Smem(LAS char* base)
      : xs(reinterpret_cast<LAS float*>(base + kLdsXs)),
        rowsum(reinterpret_cast<LAS float*>(base + kLdsRowsum)),
        route(reinterpret_cast<LAS int32_t*>(base + kLdsRoute)),
        mi(reinterpret_cast<LAS int32_t*>(base + kLdsMisc)),
        mf(reinterpret_cast<LAS float*>(base + kLdsMisc + 768)) {}
};
// misc int slots
constexpr int MI_OK = 1;         // controller -> workers: inputs ready (0: abort)
constexpr int MI_WAIT_CTR = 2;   // controller: last satisfied wait (skip repeats)
constexpr int MI_WAIT_TGT = 3;
constexpr int MI_ITEMS = 4;      // trace: items claimed by the current task
constexpr int MI_READY_LO = 6;   // trace: when the current task's first wait completed
constexpr int MI_READY_HI = 7;
constexpr int MI_XS_LAYER = 8;   // layer whose normed input xs holds (-1: none)
constexpr int MI_NEXT = 10;      // [2] claimed item indices (ping-pong)
constexpr int MI_OLD = 12;       // previous counter value of the last arrive
constexpr int MI_T_STAGED = 14;  // trace: low 32 bits of the clock when inputs were staged
constexpr int MI_T_DONE = 15;    // trace: low 32 bits of the clock when the workers finished
constexpr int MI_SCAN = 24;      // [8] block-scan scratch
constexpr int MI_TOK = 32;       // [16] token list of the current GEMV

// Routing table offsets inside Smem::route (int32 units; at most B*k <= 256 entries
// and min(E, B*k) <= 256 active experts).
constexpr int RT_IDS = 0;       // [16][16] selected experts per token
constexpr int RT_W = 256;       // [16][16] routing weights (float bits)
constexpr int RT_NACT = 512;    // number of active experts
constexpr int RT_ACT = 520;     // [256] active experts, ascending
constexpr int RT_OFF = 776;     // [257] CSR offsets of each active expert's (token, slot) list
constexpr int RT_FLAT = 1036;   // [256] b*k + j entries, experts ascending, tokens ascending

// ------------------------------------------------------------------ task context
struct Ctx {
  KParams* kp;              // kernel arguments (constant segment)
  Smem s;
  const CAS int32_t* d;     // descriptor
  int32_t task;             // global task index
  int32_t wave, lane, wi;   // wave (uniform), lane, worker index (wave - 1)
  bool ctl;                 // wave 0: the controller
};

__device__ __forceinline__ GAS uint32_t* layer_ctr(const DParams& p, int l, int off) {
  return p.counters + (int64_t)l * p.ctr.per_layer + off;
}
__device__ __forceinline__ void bar() { __syncthreads(); }

// ------------------------------------------------------------------ controller primitives
// Spin until counter >= target (lane 0 polls, then acquire).  A wait this workgroup
// already saw satisfied is skipped (counters only grow during a step).  Returns false
// when the step is aborted.  Controller wave only.
__device__ __forceinline__ bool ctl_wait(Ctx& c, GAS uint32_t* ctr, uint32_t target) {
  const DParams p = device_view(*c.kp);
  const int32_t idx = (int32_t)(ctr - p.counters);
  int ok = 1;
  if (c.lane == 0) {
    if (!(c.s.mi[MI_WAIT_CTR] == idx && target <= (uint32_t)c.s.mi[MI_WAIT_TGT])) {
      int32_t spins = 0;
      uint32_t v;
      while ((v = ctr_load(ctr)) < target) {
        if ((spins & 63) == 63 && aborted(p)) { ok = 0; break; }
        if (++spins > p.spin_limit) {
          report_error(p, 1u, c.task, idx, v, target);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      fence_acquire_agent();
      if (ok) {
        c.s.mi[MI_WAIT_CTR] = idx;
        c.s.mi[MI_WAIT_TGT] = (int32_t)target;
      }
    }
    if (ok && c.s.mi[MI_READY_LO] == 0 && c.s.mi[MI_READY_HI] == 0) {
      const uint64_t t = wall_clock64();
      c.s.mi[MI_READY_LO] = (int32_t)(uint32_t)t;
      c.s.mi[MI_READY_HI] = (int32_t)(uint32_t)(t >> 32);
    }
  }
  return __shfl(ok, 0, 64) != 0;
}

// Publish the controller's stores (written through with st_pub: waiting for their
// completion suffices) and add one to the counter; returns the old value.
__device__ __forceinline__ uint32_t ctl_arrive(Ctx& c, GAS uint32_t* ctr) {
  uint32_t old = 0;
  if (c.lane == 0) {
    wait_vm_all();
    old = ctr_add(ctr, 1u);
  }
  return (uint32_t)__shfl((int)old, 0, 64);
}

// Same, when the old value is not needed (the atomic does not wait for a reply).
__device__ __forceinline__ void ctl_signal(Ctx& c, GAS uint32_t* ctr) {
  if (c.lane == 0) {
    wait_vm_all();
    ctr_add(ctr, 1u);
  }
}

// Claim the next item of a shared queue.
__device__ __forceinline__ int32_t ctl_claim(Ctx& c, GAS uint32_t* head) {
  int32_t v = 0;
  if (c.lane == 0) {
    v = (int32_t)ctr_add(head, 1u);
    c.s.mi[MI_ITEMS] += 1;
  }
  return __shfl(v, 0, 64);
}

__device__ __forceinline__ void ctl_set_ok(Ctx& c, bool ok) {
  if (c.lane == 0) c.s.mi[MI_OK] = ok ? 1 : 0;
}
__device__ __forceinline__ int32_t read_mi(Ctx& c, int slot) { return __builtin_amdgcn_readfirstlane(c.s.mi[slot]); }
__device__ __forceinline__ bool read_ok(Ctx& c) { return read_mi(c, MI_OK) != 0; }

// ------------------------------------------------------------------ GEMV tile (workers)
// Weight rows of a tile come from up to two row segments (gate|up, or the two
// halves of a RoPE head) with a common leading dimension.
struct RowSrc {
  const GAS uint16_t* base1;
  const GAS uint16_t* base2;
  int64_t ld;
  int32_t n1;
  __device__ const GAS uint16_t* row(int i) const {
    return i < n1 ? base1 + (int64_t)i * ld : base2 + (int64_t)(i - n1) * ld;
  }
};

// Lane mapping of a K-long bf16 row onto a worker wave: LPR lanes per row, CPL
// 16-byte chunks per lane per row, RPS rows per step; worker w takes steps w, w+7, ...
// A worker walks its chunks in order f = step_index * CPL + chunk with a ring of kRing
// loads in flight per lane (kRing * 7 KB per CU): enough to stream at full HBM
// bandwidth, small enough that the queues stay short and every dependent access on
// the critical path sees a short latency.
template <int K>
struct Gemv {
  static constexpr int CH = K / 8;
  static constexpr int LPR = (CH % 64 == 0) ? 64 : (CH % 32 == 0) ? 32 : (CH % 16 == 0) ? 16 : 8;
  static constexpr int RPS = 64 / LPR;
  static constexpr int CPL = CH / LPR;
  static constexpr int MAXS = kMaxSteps;
  static constexpr int NF = MAXS * CPL;
  static constexpr int MAX_ROWS = MAXS * RPS * kWorkers;
  static_assert(K % 64 == 0, "row length must be a multiple of 64");
};

// Address of chunk f of this worker's share: row step f / CPL, 16-byte chunk f % CPL.
template <int K>
__device__ __forceinline__ const GAS void* gemv_chunk_addr(const Ctx& c, const RowSrc& src, int f) {
  using G = Gemv<K>;
  const int si = f / G::CPL, cc = f % G::CPL;
  const int row = (c.wi + kWorkers * si) * G::RPS + c.lane / G::LPR;
  const int kc = c.lane % G::LPR + G::LPR * cc;
  return src.row(row) + kc * 8;
}

// Worker side of a GEMV tile (includes the task's two barriers).  The worker's F chunks
// (its row steps w, w+7, ... times CPL) stream through a ring of kRing loads: the first
// kRing are issued before the first barrier (weight prefetch while the controller waits
// for the inputs), the rest as chunks are consumed.  Every ring slot issues exactly one
// load per round (slots past F load a small cached dummy line), so the loop body is
// straight-line and the wait-counter pass keeps kRing loads in flight.
// rowsum[row * nb + j] = W[row] . x_j, x_j = xs + tok[j] * K, rows < R.  NB bounds nb.
template <int K, int NB>
__device__ __forceinline__ bool gemv_tile(const Ctx& c, const RowSrc& src, int R, const LAS float* xs,
                                          const LAS int32_t* tok, int nb, LAS float* rowsum,
                                          const GAS u32x4* dummy) {
  using G = Gemv<K>;
  const int S = (R + G::RPS - 1) / G::RPS;
  const int ns = c.wi < S ? (S - c.wi + kWorkers - 1) / kWorkers : 0;
  const int F = ns * G::CPL;
  const GAS void* dum = dummy + c.lane;
  u32x4 ring[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) ring[r] = ld_stream16(r < F ? gemv_chunk_addr<K>(c, src, r) : dum);
  bar();
  if (!read_ok(const_cast<Ctx&>(c))) return false;
  float acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = 0.0f;
  for (int base = 0; base < F; base += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int f = base + r;
      const u32x4 w = ring[r];
      const int fn = f + kRing;
      ring[r] = ld_stream16(fn < F ? gemv_chunk_addr<K>(c, src, fn) : dum);
      if (f < F) {
        const int cc = f % G::CPL;
        const int kc = c.lane % G::LPR + G::LPR * cc;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (NB == 1 || j < nb) {
            const LAS f32x4* xp = reinterpret_cast<const LAS f32x4*>(xs + tok[j] * K + kc * 8);
            acc[j] += dot8(w, xp[0], xp[1]);
          }
        }
        if (cc == G::CPL - 1) {
          const int row = (c.wi + kWorkers * (f / G::CPL)) * G::RPS + c.lane / G::LPR;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if (NB == 1 || j < nb) {
              const float t = group_sum<G::LPR>(acc[j]);
              if (c.lane % G::LPR == 0 && row < R) rowsum[row * nb + j] = t;
              acc[j] = 0.0f;
            }
          }
        }
      }
    }
  }
  bar();
  return true;
}

template <int K>
__device__ __forceinline__ bool worker_gemv(const Ctx& c, const RowSrc& src, int R, const LAS float* xs,
                                            const LAS int32_t* tok, int nb, LAS float* rowsum) {
  const GAS u32x4* dummy = (const GAS u32x4*)c.kp->dummy;
  if (nb == 1) return gemv_tile<K, 1>(c, src, R, xs, tok, nb, rowsum, dummy);
  return gemv_tile<K, kMaxBatch>(c, src, R, xs, tok, nb, rowsum, dummy);
}

// Controller side of the same two barriers.
__device__ __forceinline__ bool ctl_gemv_barriers(Ctx& c, bool ok) {
  ctl_set_ok(c, ok);
  if (c.lane == 0 && c.s.mi[MI_T_STAGED] == 0) c.s.mi[MI_T_STAGED] = (int32_t)(uint32_t)wall_clock64();
  bar();
  if (!ok) return false;
  bar();
  if (c.lane == 0 && c.s.mi[MI_T_DONE] == 0) c.s.mi[MI_T_DONE] = (int32_t)(uint32_t)wall_clock64();
  return true;
}

// ------------------------------------------------------------------ activation staging (controller)
// xs[b][k] = h_l[b][k] * inv_rms_b * gamma_l[k] for every token of the batch: the RMSNorm
// that every consumer of layer l's input applies on the fly.  inv_rms_b comes from the
// per-row-tile sums of squares written when the residual rows were finalised.  The
// staged vector is kept while the next tasks on this CU read the same layer's input.
__device__ __forceinline__ void ctl_stage_x_normed(Ctx& c, int l) {
  if (read_mi(c, MI_XS_LAYER) == l) return;
  const DParams p = device_view(*c.kp);
  const int B = p.batch, H = p.hidden, NRT = p.shape.n_rt;
  float part[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    float t = 0.0f;
    if (b < B)
      for (int r = c.lane; r < NRT; r += 64) t += p.ss[((int64_t)l * p.max_batch + b) * NRT + r];
    part[b] = t;
  }
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    if (b < B) {
      const float t = group_sum<64>(part[b]);
      if (c.lane == 0) c.s.mf[b] = 1.0f / sqrtf(t / (float)H + p.rms_eps);
    }
  }
  const GAS uint16_t* gamma = p.norm + (int64_t)l * H;
  const int n8 = B * (H / 8);
#pragma unroll 4
  for (int i = c.lane; i < n8; i += 64) {
    const int b = i / (H / 8), k8 = (i % (H / 8)) * 8;
    const GAS float* hp = p.h + ((int64_t)l * p.max_batch + b) * H + k8;
    const f32x4 h0 = *reinterpret_cast<const GAS f32x4*>(hp);
    const f32x4 h1 = *reinterpret_cast<const GAS f32x4*>(hp + 4);
    const u32x4 gw = *reinterpret_cast<const GAS u32x4*>(gamma + k8);
    const float r = c.s.mf[b];
    f32x4 o0, o1;
    o0.x = h0.x * r * bf_lo(gw.x); o0.y = h0.y * r * bf_hi(gw.x);
    o0.z = h0.z * r * bf_lo(gw.y); o0.w = h0.w * r * bf_hi(gw.y);
    o1.x = h1.x * r * bf_lo(gw.z); o1.y = h1.y * r * bf_hi(gw.z);
    o1.z = h1.z * r * bf_lo(gw.w); o1.w = h1.w * r * bf_hi(gw.w);
    LAS float* xo = c.s.xs + b * H + k8;
    *reinterpret_cast<LAS f32x4*>(xo) = o0;
    *reinterpret_cast<LAS f32x4*>(xo + 4) = o1;
  }
  if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
  if (c.lane == 0) c.s.mi[MI_XS_LAYER] = l;
}

// Stage nb rows of K floats from global memory (row stride `stride`) into xs.
template <int K>
__device__ __forceinline__ void ctl_stage_rows(Ctx& c, const GAS float* src, int64_t stride, int nb) {
  for (int i = c.lane; i < nb * (K / 4); i += 64) {
    const int b = i / (K / 4), k4 = (i % (K / 4)) * 4;
    *reinterpret_cast<LAS f32x4*>(c.s.xs + b * K + k4) = *reinterpret_cast<const GAS f32x4*>(src + b * stride + k4);
  }
  if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
  if (c.lane == 0) c.s.mi[MI_XS_LAYER] = -1;
}

// ------------------------------------------------------------------ residual finalisation (controller)
// The fused residual add + RMSNorm at the end of a layer ("Where the speedup comes
// from": parallel layers are rejoined only by it).  The last arriver of residual row
// tile rt writes h_{l+1} = h_l + sum_g a_g + sum_ds m_ds for those rows and their sum of
// squares; consumers of layer l+1 normalise on the fly.
__device__ __forceinline__ void ctl_finalize_rows(Ctx& c, int l, int rt) {
  const DParams p = device_view(*c.kp);
  fence_acquire_agent();
  const int R = p.shape.rt_rows, H = p.hidden, B = p.batch;
  const int r0 = rt * R;
  const int64_t hstride = (int64_t)p.max_batch * H;
  LAS float* red = c.s.rowsum;  // [B][R] squares (the tile's row sums are consumed)
  for (int i = c.lane; i < B * R; i += 64) {
    const int b = i / R, r = r0 + i % R;
    const int64_t hb = (int64_t)b * H + r;
    float v = p.h[(int64_t)l * hstride + hb];
    for (int g0 = 0; g0 < p.n_kv; g0 += 4) {
      float t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        t[j] = g0 + j < p.n_kv ? p.a_part[((int64_t)l * p.n_kv + g0 + j) * hstride + hb] : 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) v += t[j];
    }
    for (int d0 = 0; d0 < p.shape.n_ds; d0 += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        t[j] = d0 + j < p.shape.n_ds ? p.m_part[((int64_t)l * p.shape.n_ds + d0 + j) * hstride + hb] : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) v += t[j];
    }
    st_pub(p.h + (int64_t)(l + 1) * hstride + hb, v);
    red[i] = v * v;
  }
  for (int b = 0; b < B; ++b) {
    float t = 0.0f;
    for (int r = c.lane; r < R; r += 64) t += red[b * R + r];
    t = group_sum<64>(t);
    if (c.lane == 0) st_pub(p.ss + ((int64_t)(l + 1) * p.max_batch + b) * p.shape.n_rt + rt, t);
  }
  ctl_signal(c, layer_ctr(p, l + 1, p.ctr.x_ready));
}

// Arrive on a residual row tile; the last of its n_kv + n_ds producers finalises it.
__device__ __forceinline__ void ctl_arrive_rt(Ctx& c, int l, int rt) {
  const DParams p = device_view(*c.kp);
  const uint32_t old = ctl_arrive(c, layer_ctr(p, l, p.ctr.rt + rt));
  if (old + 1 == (uint32_t)(p.n_kv + p.shape.n_ds)) ctl_finalize_rows(c, l, rt);
}

// ------------------------------------------------------------------ OP_EMBED (controller)
// h_0 rows of residual tile rt (token embeddings, widened to fp32) and their sums of
// squares; the task of tile 0 also writes this step's RoPE table (cos, sin of
// position * base^(-2i/hd), angles in fp64) for the QKV epilogues of every layer.
__device__ __forceinline__ bool op_embed(Ctx& c) {
  if (!c.ctl) return true;
  const DParams p = device_view(*c.kp);
  const int rt = c.d[D_ARG0];
  const int R = p.shape.rt_rows, H = p.hidden, B = p.batch;
  LAS float* red = c.s.rowsum;
  for (int i = c.lane; i < B * R; i += 64) {
    const int b = i / R, r = rt * R + i % R;
    int tok = p.tokens[b];
    if (tok < 0 || tok >= p.vocab) {
      report_error(p, 2u, c.task, -1, (uint32_t)tok, (uint32_t)p.vocab);
      tok = 0;
    }
    const float v = bf16_to_f32(p.embed[(int64_t)tok * H + r]);
    st_pub(p.h + (int64_t)b * H + r, v);
    red[i] = v * v;
  }
  for (int b = 0; b < B; ++b) {
    float t = 0.0f;
    for (int r = c.lane; r < R; r += 64) t += red[b * R + r];
    t = group_sum<64>(t);
    if (c.lane == 0) st_pub(p.ss + (int64_t)b * p.shape.n_rt + rt, t);
  }
  if (rt == 0) {
    const int half = p.head_dim / 2;
    for (int i = c.lane; i < B * half; i += 64) {
      const int b = i / half, k = i % half;
      const double ang = (double)p.seq_lens[b] * p.inv_freq[k];
      st_pub(p.rope + 2 * i, (float)cos(ang));
      st_pub(p.rope + 2 * i + 1, (float)sin(ang));
    }
  }
  ctl_signal(c, layer_ctr(p, 0, p.ctr.x_ready));
  return true;
}

// ------------------------------------------------------------------ OP_QKV
// Tile = head hh of the q|k|v rows, dims [j0, j0+PB) and [j0+hd/2, j0+hd/2+PB), so every
// RoPE pair (i, i+hd/2) is in the tile.  Epilogue: RoPE at the token's position, q to the
// workspace, k and v as bf16 into the paged-KV slot (page_table[b][pos/page], pos%page)
// of this layer (K pages token-major, V pages dim-major).
template <int K>
__device__ __forceinline__ bool op_qkv(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], hh = c.d[D_ARG0], j0 = c.d[D_ARG1], PB = c.d[D_ARG2];
  const int hd = p.head_dim, half = hd / 2, H = p.hidden, B = p.batch;
  const GAS uint16_t* wl = p.w_qkv + (int64_t)l * (p.n_q + 2 * p.n_kv) * hd * H;
  const RowSrc src{wl + ((int64_t)hh * hd + j0) * H, wl + ((int64_t)hh * hd + half + j0) * H, H, PB};
  if (!c.ctl) {
    return worker_gemv<K>(c, src, 2 * PB, c.s.xs, c.s.mi + MI_TOK, B, c.s.rowsum);
  } else {
    const bool ok = ctl_wait(c, p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET]);
    if (ok) ctl_stage_x_normed(c, l);
    if (!ctl_gemv_barriers(c, ok)) return false;
    for (int i = c.lane; i < PB * B; i += 64) {
      const int r = i / B, b = i % B, dim = j0 + r;
      const float a = c.s.rowsum[r * B + b], bb = c.s.rowsum[(PB + r) * B + b];
      const int pos = p.seq_lens[b];
      float o1 = a, o2 = bb;
      if (hh < p.n_q + p.n_kv) {
        const float cs = p.rope[((int64_t)b * half + dim) * 2], sn = p.rope[((int64_t)b * half + dim) * 2 + 1];
        o1 = a * cs - bb * sn;
        o2 = bb * cs + a * sn;
      }
      if (hh < p.n_q) {
        GAS float* q = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * hd + (int64_t)hh * hd;
        st_pub(q + dim, o1);
        st_pub(q + dim + half, o2);
      } else {
        const int lp = pos / p.page, t = pos % p.page;
        const int phys = (lp < p.max_pages) ? p.page_table[(int64_t)b * p.max_pages + lp] : -1;
        if (phys < 0 || phys >= p.n_pages) {
          report_error(p, 2u, c.task, -1, (uint32_t)phys, (uint32_t)p.n_pages);
          continue;
        }
        const bool is_k = hh < p.n_q + p.n_kv;
        const int g = is_k ? hh - p.n_q : hh - p.n_q - p.n_kv;
        const int64_t pg = (((int64_t)l * 2 + (is_k ? 0 : 1)) * p.n_pages + phys) * p.n_kv + g;
        GAS uint16_t* base = p.kv_pool + pg * (int64_t)p.page * hd;
        if (is_k) {
          st_pub(base + (int64_t)t * hd + dim, f32_to_bf16(o1));
          st_pub(base + (int64_t)t * hd + dim + half, f32_to_bf16(o2));
        } else {
          st_pub(base + (int64_t)dim * p.page + t, f32_to_bf16(o1));
          st_pub(base + (int64_t)(dim + half) * p.page + t, f32_to_bf16(o2));
        }
      }
    }
    ctl_signal(c, p.counters + c.d[D_SIGNAL]);
  }
  return true;
}

// ------------------------------------------------------------------ OP_ROUTER / OP_LM_HEAD
// Plain GEMV tiles on the normed input: router logits (layer l) or vocabulary logits
// (final norm, tied embedding).
template <int K>
__device__ __forceinline__ bool op_rows_on_x(Ctx& c, bool lm_head) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], r0 = c.d[D_ARG0], R = c.d[D_ARG1];
  const int H = p.hidden, B = p.batch;
  const GAS uint16_t* base = lm_head ? p.embed + (int64_t)r0 * H : p.w_router + ((int64_t)l * p.n_experts + r0) * H;
  const RowSrc src{base, base, H, R};
  if (!c.ctl) {
    return worker_gemv<K>(c, src, R, c.s.xs, c.s.mi + MI_TOK, B, c.s.rowsum);
  } else {
    const bool ok = ctl_wait(c, p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET]);
    if (ok) ctl_stage_x_normed(c, l);
    if (!ctl_gemv_barriers(c, ok)) return false;
    for (int i = c.lane; i < R * B; i += 64) {
      const int r = i / B, b = i % B;
      if (lm_head) p.logits[(int64_t)b * p.vocab + r0 + r] = c.s.rowsum[i];
      else st_pub(p.router + ((int64_t)l * p.max_batch + b) * p.n_experts + r0 + r, c.s.rowsum[i]);
    }
    if (c.d[D_SIGNAL] >= 0) ctl_signal(c, p.counters + c.d[D_SIGNAL]);
  }
  return true;
}

// ------------------------------------------------------------------ OP_OPROJ
// Split-K over KV groups (Figure 7: the O-proj of a KV group starts as soon as that
// group's attention output lands): rows [rt*R, +R) of W_o, columns of group g.
template <int K>
__device__ __forceinline__ bool op_oproj(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], rt = c.d[D_ARG0], g = c.d[D_ARG1];
  const int R = p.shape.rt_rows, H = p.hidden, KO = p.n_q * p.head_dim, B = p.batch;
  const GAS uint16_t* base = p.w_o + ((int64_t)l * H + (int64_t)rt * R) * KO + (int64_t)g * K;
  const RowSrc src{base, base, KO, R};
  if (!c.ctl) {
    return worker_gemv<K>(c, src, R, c.s.xs, c.s.mi + MI_TOK, B, c.s.rowsum);
  } else {
    const bool ok = ctl_wait(c, p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET]);
    if (ok) ctl_stage_rows<K>(c, p.attn_o + (int64_t)l * p.max_batch * KO + (int64_t)g * K, KO, B);
    if (!ctl_gemv_barriers(c, ok)) return false;
    for (int i = c.lane; i < R * B; i += 64) {
      const int r = i / B, b = i % B;
      st_pub(p.a_part + (((int64_t)l * p.n_kv + g) * p.max_batch + b) * H + rt * R + r, c.s.rowsum[i]);
    }
    ctl_arrive_rt(c, l, rt);
  }
  return true;
}

// ------------------------------------------------------------------ routing (all waves)
// Exclusive prefix sum of one int per thread over the workgroup; total receives the sum.
__device__ __forceinline__ int block_exscan(int v, LAS int32_t* tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  bar();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = tmp[i];
    pre += i < w ? t : 0;
    tot += t;
  }
  bar();
  total = tot;
  return pre + x - v;
}

// ROUTER_TOPK + ROUTE_FINALIZE + MOE_GATHER in LDS: top-k of each token's router logits
// (descending, ties to the lower expert index), softmax over the selected logits, then
// the active experts in ascending order and, per expert, its (token, slot) entries in
// ascending token order.  Called by every wave after the controller's acquire of the
// router counter; no wave has weight loads in flight here.
__device__ __forceinline__ void route_layer(Ctx& c, int l, bool write_debug) {
  const DParams p = device_view(*c.kp);
  const int B = p.batch, E = p.n_experts, k = p.top_k;
  LAS int32_t* rt = c.s.route;
  LAS float* rw = reinterpret_cast<LAS float*>(rt + RT_W);
  const int lane = c.lane;
  for (int b = c.wave; b < B; b += kWaves) {
    const GAS float* r = p.router + ((int64_t)l * p.max_batch + b) * E;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? r[e] : -INFINITY;
    }
    float sel_v0 = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (lane + 64 * i == bi) v[i] = -INFINITY;
      if (j == 0) sel_v0 = bv;
      if (lane == 0) {
        rt[RT_IDS + b * 16 + j] = bi;
        rw[b * 16 + j] = bv;  // logit for now
      }
    }
    if (lane == 0) {
      float sum = 0.0f;
      for (int j = 0; j < k; ++j) {
        const float ex = expf(rw[b * 16 + j] - sel_v0);
        rw[b * 16 + j] = ex;
        sum += ex;
      }
      for (int j = 0; j < k; ++j) rw[b * 16 + j] /= sum;
    }
  }
  bar();
  // per-expert entry counts, one thread per expert, then block-wide exclusive scans give
  // each active expert its rank and its offset in the flat (token, slot) list.
  const int e = threadIdx.x;
  int m_e = 0;
  if (e < E)
    for (int b = 0; b < B; ++b)
      for (int j = 0; j < k; ++j) m_e += rt[RT_IDS + b * 16 + j] == e;
  int n_entries = 0, n_act = 0;
  const int off = block_exscan(m_e, c.s.mi + MI_SCAN, n_entries);
  const int rank = block_exscan(m_e > 0 ? 1 : 0, c.s.mi + MI_SCAN, n_act);
  if (m_e > 0) {
    rt[RT_ACT + rank] = e;
    rt[RT_OFF + rank] = off;
    int at = off;
    for (int b = 0; b < B; ++b)
      for (int j = 0; j < k; ++j)
        if (rt[RT_IDS + b * 16 + j] == e) rt[RT_FLAT + at++] = b * k + j;
  }
  if (threadIdx.x == 0) {
    rt[RT_OFF + n_act] = n_entries;
    rt[RT_NACT] = n_act;
  }
  if (write_debug && threadIdx.x < B * k) {
    const int b = threadIdx.x / k, j = threadIdx.x % k;
    p.topk_ids[((int64_t)l * p.max_batch + b) * k + j] = rt[RT_IDS + b * 16 + j];
    p.topk_w[((int64_t)l * p.max_batch + b) * k + j] = rw[b * 16 + j];
  }
  bar();
}

// ------------------------------------------------------------------ OP_MOE_UP (claimer)
// Claims (active expert, tile of up_rows activation rows); weights = up_rows gate rows and
// the matching up rows; epilogue silu(gate) * up for every token routed to the expert;
// arrives on the expert's up counter.
template <int K>
__device__ __forceinline__ bool op_moe_up(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  const int UR = p.shape.up_rows, NT = p.shape.n_up_tiles, H = p.hidden, I = p.inter, k = p.top_k;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.up_claim);
  if (c.ctl) {
    const bool ok = ctl_wait(c, p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET]);
    if (ok) {
      ctl_stage_x_normed(c, l);
      const int32_t first = ctl_claim(c, head);
      if (c.lane == 0) c.s.mi[MI_NEXT] = first;
    }
    ctl_set_ok(c, ok);
  }
  bar();
  if (!read_ok(c)) return false;
  route_layer(c, l, c.d[D_ARG0] == 0);
  const LAS int32_t* rt = c.s.route;
  const int n_items = __builtin_amdgcn_readfirstlane(rt[RT_NACT]) * NT;
  for (int j = 0;; ++j) {
    const int idx = read_mi(c, MI_NEXT + (j & 1));
    if (idx >= n_items) break;
    const int a = idx / NT, tile = idx % NT;
    const int e = __builtin_amdgcn_readfirstlane(rt[RT_ACT + a]);
    const int o0 = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a]);
    const int n_e = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a + 1]) - o0;
    const GAS uint16_t* base = p.w_gate_up + (((int64_t)l * p.n_experts + e) * 2 * I + (int64_t)tile * UR) * H;
    const RowSrc src{base, base + (int64_t)I * H, H, UR};
    if (!c.ctl) {
      if (!worker_gemv<K>(c, src, 2 * UR, c.s.xs, c.s.mi + MI_TOK, n_e, c.s.rowsum)) return false;
    } else {
      if (c.lane < n_e) c.s.mi[MI_TOK + c.lane] = rt[RT_FLAT + o0 + c.lane] / k;
      const int32_t nxt = ctl_claim(c, head);
      if (c.lane == 0) c.s.mi[MI_NEXT + ((j + 1) & 1)] = nxt;
      if (!ctl_gemv_barriers(c, true)) return false;
      for (int i = c.lane; i < UR * n_e; i += 64) {
        const int r = i / n_e, jj = i % n_e;
        const float gt = c.s.rowsum[r * n_e + jj], u = c.s.rowsum[(UR + r) * n_e + jj];
        const float act = gt / (1.0f + expf(-gt)) * u;
        const int slot = rt[RT_FLAT + o0 + jj];  // b * k + j
        st_pub(p.moe_act + ((int64_t)l * p.max_batch * k + slot) * I + (int64_t)tile * UR + r, act);
      }
      ctl_signal(c, layer_ctr(p, l, p.ctr.up_done + e));
      if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
    }
  }
  return true;
}

// ------------------------------------------------------------------ OP_MOE_DOWN (claimer)
// Claims (residual row tile rt, expert split ds): for each active expert of the split
// (every n_ds-th in ascending order) the workers stream W_down[e][rows of rt] while the
// controller waits for that expert's up tiles and stages its activations; y_e is
// weighted by the router scores into the split's partial m_ds[b][rows]; the last
// producer of the row tile finalises the residual.
template <int K>
__device__ __forceinline__ bool op_moe_down(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  const int R = p.shape.rt_rows, NDS = p.shape.n_ds, H = p.hidden, I = p.inter, B = p.batch, k = p.top_k;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.down_claim);
  if (c.ctl) {
    const bool ok = ctl_wait(c, p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET]);
    if (ok) {
      const int32_t first = ctl_claim(c, head);
      if (c.lane == 0) c.s.mi[MI_NEXT] = first;
      if (c.lane == 0) c.s.mi[MI_XS_LAYER] = -1;
    }
    ctl_set_ok(c, ok);
  }
  bar();
  if (!read_ok(c)) return false;
  route_layer(c, l, false);
  const LAS int32_t* rt = c.s.route;
  const LAS float* rw = reinterpret_cast<const LAS float*>(rt + RT_W);
  const int n_act = __builtin_amdgcn_readfirstlane(rt[RT_NACT]);
  LAS float* macc = c.s.rowsum + 1024;  // [R][B], controller only
  for (int j = 0;; ++j) {
    const int idx = read_mi(c, MI_NEXT + (j & 1));
    if (idx >= p.shape.n_rt * NDS) break;
    const int rtile = idx / NDS, ds = idx % NDS;
    if (c.ctl) {
      for (int i = c.lane; i < R * B; i += 64) macc[i] = 0.0f;
      const int32_t nxt = ctl_claim(c, head);
      if (c.lane == 0) c.s.mi[MI_NEXT + ((j + 1) & 1)] = nxt;
    }
    for (int a = ds; a < n_act; a += NDS) {
      const int e = __builtin_amdgcn_readfirstlane(rt[RT_ACT + a]);
      const int o0 = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a]);
      const int n_e = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a + 1]) - o0;
      const GAS uint16_t* base = p.w_down + (((int64_t)l * p.n_experts + e) * H + (int64_t)rtile * R) * I;
      const RowSrc src{base, base, I, R};
      if (!c.ctl) {
        if (!worker_gemv<K>(c, src, R, c.s.xs, c.s.mi + MI_TOK, n_e, c.s.rowsum)) return false;
      } else {
        const bool ok = ctl_wait(c, layer_ctr(p, l, p.ctr.up_done + e), (uint32_t)p.shape.n_up_tiles);
        if (ok) {
          for (int i = c.lane; i < n_e * (K / 4); i += 64) {
            const int jj = i / (K / 4), k4 = (i % (K / 4)) * 4;
            const int slot = rt[RT_FLAT + o0 + jj];
            *reinterpret_cast<LAS f32x4*>(c.s.xs + jj * K + k4) =
                *reinterpret_cast<const GAS f32x4*>(p.moe_act + ((int64_t)l * p.max_batch * k + slot) * I + k4);
          }
          if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
        }
        if (!ctl_gemv_barriers(c, ok)) return false;
        for (int i = c.lane; i < R * n_e; i += 64) {
          const int r = i / n_e, jj = i % n_e;
          const int slot = rt[RT_FLAT + o0 + jj];
          const int b = slot / k, sj = slot % k;
          macc[r * B + b] += rw[b * 16 + sj] * c.s.rowsum[r * n_e + jj];
        }
      }
    }
    if (c.ctl) {
      for (int i = c.lane; i < R * B; i += 64) {
        const int r = i / B, b = i % B;
        st_pub(p.m_part + (((int64_t)l * NDS + ds) * p.max_batch + b) * H + (int64_t)rtile * R + r, macc[i]);
      }
      ctl_arrive_rt(c, l, rtile);
    }
    bar();  // the next claimed index is published
  }
  return true;
}

// ------------------------------------------------------------------ OP_ATTN (claimer)
// Paged GQA decode attention, split over pages ("Tasks": ATTN_DECODE over a partial KV
// slice, ATTN_COMBINE merging the partials; ATTN_DRAIN claiming from the queue).  One
// item = (sequence b, KV group g, chunk of pages_per_item pages); worker w takes every
// 7th page of the chunk.  Per 16-token page:
//   S^T[t][h] = K[t][:] . Qs^T[:][h]   (v_mfma_f32_16x16x32_bf16, tokens x heads,
//                                        Qs = q * log2(e)/sqrt(hd) in bf16)
//   online softmax in base 2 per head, P in bf16
//   O^T[d][h] += V^T[d][t] P^T[t][h]    (v_mfma_f32_16x16x16_bf16; V pages are stored
//                                        dim-major so V^T rows are contiguous)
// The cached pages are streamed before the controller's wait for this layer's QKV
// tiles; only the page holding the new token is read after it.  The last item of a
// (sequence, group) merges all chunks (log-sum-exp) with every wave.
__device__ __forceinline__ void attn_map(const DParams& p, int idx, int& b, int& g, int& chunk, int& nchunks,
                                         int& base_bg) {
  const int ppi = p.shape.pages_per_item;
  b = -1;
  int acc = 0;
  for (int bb = 0; bb < p.batch; ++bb) {
    const int npg = p.seq_lens[bb] / p.page + 1;
    const int nit = (npg + ppi - 1) / ppi;
    if (idx < acc + nit * p.n_kv) {
      const int local = idx - acc;
      b = bb;
      g = local / nit;
      chunk = local % nit;
      nchunks = nit;
      base_bg = acc + g * nit;
      return;
    }
    acc += nit * p.n_kv;
  }
}

template <int HD>
__device__ __forceinline__ bool op_attn(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  const int nkv = p.n_kv, ppi = p.shape.pages_per_item, hpg = p.n_q / nkv;
  constexpr int NK = HD / 32, NV = HD / 16, MAXP = kMaxPagesPerWave;
  int n_items = 0;
  for (int b = 0; b < p.batch; ++b) n_items += ((p.seq_lens[b] / p.page + 1 + ppi - 1) / ppi) * nkv;
  if (n_items > p.max_attn_items) n_items = p.max_attn_items;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.attn_claim);
  LAS float* qs = c.s.xs;                              // [hpg][HD] fp32 queries
  LAS float* mw = c.s.xs + 16 * HD;                    // [7][16] running max per worker
  LAS float* lw = mw + kWorkers * 16;                  // [7][16] running sum
  LAS float* ow = lw + kWorkers * 16;                  // [7][hpg][HD] unnormalised outputs
  LAS float* part = ow + kWorkers * 16 * HD;           // [hpg][HD + 2] merged partial
  bool waited = false;
  if (c.ctl) {
    const int32_t first = ctl_claim(c, head);
    if (c.lane == 0) {
      c.s.mi[MI_NEXT] = first;
      c.s.mi[MI_XS_LAYER] = -1;
    }
  }
  bar();
  for (int j = 0;; ++j) {
    const int idx = read_mi(c, MI_NEXT + (j & 1));
    if (idx >= n_items) break;
    int b, g = 0, chunk = 0, nchunks = 0, base_bg = 0;
    attn_map(p, idx, b, g, chunk, nchunks, base_bg);
    const int pos = p.seq_lens[b];
    const int npg = pos / p.page + 1, last = npg - 1;
    const int c0 = chunk * ppi, c1 = min(npg, c0 + ppi);
    u32x4 kr[MAXP][NK];
    u32x2 vr[MAXP][NV];
    int lp[MAXP];
    int64_t kbase[MAXP], vbase[MAXP];
    if (!c.ctl) {
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        lp[i] = c0 + c.wi + kWorkers * i;
        kbase[i] = 0;
        vbase[i] = 0;
        if (lp[i] < c1) {
          const int phys = lp[i] < p.max_pages ? p.page_table[(int64_t)b * p.max_pages + lp[i]] : -1;
          if (phys < 0 || phys >= p.n_pages) {
            if (c.lane == 0) report_error(p, 2u, c.task, -1, (uint32_t)phys, (uint32_t)p.n_pages);
            lp[i] = c1;  // skip
          } else {
            kbase[i] = ((((int64_t)l * 2 + 0) * p.n_pages + phys) * nkv + g) * (int64_t)p.page * HD;
            vbase[i] = ((((int64_t)l * 2 + 1) * p.n_pages + phys) * nkv + g) * (int64_t)p.page * HD;
          }
        }
        if (lp[i] < c1 && lp[i] != last) {
#pragma unroll
          for (int kk = 0; kk < NK; ++kk)
            kr[i][kk] = ld_stream16(p.kv_pool + kbase[i] + (c.lane & 15) * HD + kk * 32 + (c.lane >> 4) * 8);
#pragma unroll
          for (int dt = 0; dt < NV; ++dt)
            vr[i][dt] = ld_stream8(p.kv_pool + vbase[i] + (dt * 16 + (c.lane & 15)) * 16 + (c.lane >> 4) * 4);
        }
      }
    } else {
      bool ok = true;
      if (!waited) {
        ok = ctl_wait(c, p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET]);
        waited = true;
      }
      if (ok) {
        const GAS float* qsrc = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * HD + (int64_t)g * hpg * HD;
        for (int i = c.lane; i < hpg * HD / 4; i += 64)
          *reinterpret_cast<LAS f32x4*>(qs + i * 4) = *reinterpret_cast<const GAS f32x4*>(qsrc + i * 4);
        const int32_t nxt = ctl_claim(c, head);
        if (c.lane == 0) c.s.mi[MI_NEXT + ((j + 1) & 1)] = nxt;
      }
      ctl_set_ok(c, ok);
    }
    bar();
    if (!read_ok(c)) return false;
    if (!c.ctl) {
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        if (lp[i] < c1 && lp[i] == last) {
#pragma unroll
          for (int kk = 0; kk < NK; ++kk)
            kr[i][kk] = *reinterpret_cast<const GAS u32x4*>(p.kv_pool + kbase[i] + (c.lane & 15) * HD + kk * 32 +
                                                            (c.lane >> 4) * 8);
#pragma unroll
          for (int dt = 0; dt < NV; ++dt)
            vr[i][dt] = *reinterpret_cast<const GAS u32x2*>(p.kv_pool + vbase[i] + (dt * 16 + (c.lane & 15)) * 16 +
                                                            (c.lane >> 4) * 4);
        }
      }
      // Q^T operand: lane holds head (lane & 15), dims kk*32 + (lane>>4)*8 + [0, 8)
      const int hq = c.lane & 15;
      const float qscale = 1.4426950408889634f / sqrtf((float)HD);
      u32x4 qb[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (hq < hpg) {
          const LAS float* qp = qs + hq * HD + kk * 32 + (c.lane >> 4) * 8;
          const f32x4 a0 = *reinterpret_cast<const LAS f32x4*>(qp);
          const f32x4 a1 = *reinterpret_cast<const LAS f32x4*>(qp + 4);
          qb[kk] = u32x4{pack_bf16x2(a0.x * qscale, a0.y * qscale), pack_bf16x2(a0.z * qscale, a0.w * qscale),
                         pack_bf16x2(a1.x * qscale, a1.y * qscale), pack_bf16x2(a1.z * qscale, a1.w * qscale)};
        } else {
          qb[kk] = u32x4{0, 0, 0, 0};
        }
      }
      float m = -INFINITY, lsum = 0.0f;
      f32x4 o[NV];
#pragma unroll
      for (int dt = 0; dt < NV; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        if (lp[i] >= c1) continue;
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[i][kk]),
                                                      __builtin_bit_cast(bf16x8, qb[kk]), s, 0, 0, 0);
        if (lp[i] == last) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (lp[i] * p.page + (c.lane >> 4) * 4 + r > pos) s[r] = -INFINITY;
        }
        float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
        pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
        const float mn = fmaxf(m, pm);
        const float alpha = exp2f(m - mn);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2f(s[r] - mn);
        float ps = (pr[0] + pr[1]) + (pr[2] + pr[3]);
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        lsum = lsum * alpha + ps;
        m = mn;
        const u32x2 pb2 = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
        const s16x4 pb = __builtin_bit_cast(s16x4, pb2);
#pragma unroll
        for (int dt = 0; dt < NV; ++dt) {
          o[dt] *= alpha;
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vr[i][dt]), pb, o[dt], 0, 0, 0);
        }
      }
      if (c.lane < 16) {
        mw[c.wi * 16 + c.lane] = m;
        lw[c.wi * 16 + c.lane] = lsum;
      }
      if (hq < hpg) {
#pragma unroll
        for (int dt = 0; dt < NV; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) ow[(c.wi * hpg + hq) * HD + dt * 16 + (c.lane >> 4) * 4 + r] = o[dt][r];
      }
    }
    bar();
    // merge the workers: unnormalised o, running max M and sum L per head (all waves)
    for (int t = threadIdx.x; t < hpg * HD; t += kThreads) {
      const int h = t / HD, dd = t % HD;
      float M = -INFINITY;
      for (int ww = 0; ww < kWorkers; ++ww) M = fmaxf(M, mw[ww * 16 + h]);
      float acc = 0.0f, L = 0.0f;
      for (int ww = 0; ww < kWorkers; ++ww) {
        const float sc = exp2f(mw[ww * 16 + h] - M);
        acc += sc * ow[(ww * hpg + h) * HD + dd];
        L += sc * lw[ww * 16 + h];
      }
      part[h * (HD + 2) + dd] = acc;
      if (dd == 0) {
        part[h * (HD + 2) + HD] = M;
        part[h * (HD + 2) + HD + 1] = L;
      }
    }
    bar();
    if (c.ctl) {
      GAS float* dst = p.attn_part + (int64_t)idx * hpg * (HD + 2);
      for (int i = c.lane; i < hpg * (HD + 2); i += 64) st_pub(dst + i, part[i]);
      const uint32_t old = ctl_arrive(c, layer_ctr(p, l, p.ctr.attn_items + b * nkv + g));
      if (c.lane == 0) c.s.mi[MI_OLD] = (int32_t)old;
    }
    bar();
    if ((uint32_t)read_mi(c, MI_OLD) + 1 == (uint32_t)nchunks) {
      // last item of (b, g): combine all chunks (log-sum-exp merge, chunk order fixed)
      fence_acquire_agent();
      const GAS float* pb = p.attn_part + (int64_t)base_bg * hpg * (HD + 2);
      LAS float* scl = c.s.xs;                         // [nchunks][hpg] merged weights
      LAS float* mrow = c.s.xs + kAttnMaxChunks * 16;  // [hpg] inverse denominators
      for (int h = c.wave; h < hpg; h += kWaves) {
        float M = -INFINITY;
        for (int ci = c.lane; ci < nchunks; ci += 64) M = fmaxf(M, pb[((int64_t)ci * hpg + h) * (HD + 2) + HD]);
        M = wave_max(M);
        float den = 0.0f;
        for (int ci = c.lane; ci < nchunks; ci += 64) {
          const GAS float* pc = pb + ((int64_t)ci * hpg + h) * (HD + 2);
          const float sc = exp2f(pc[HD] - M);
          scl[ci * hpg + h] = sc;
          den += sc * pc[HD + 1];
        }
        den = group_sum<64>(den);
        if (c.lane == 0) mrow[h] = 1.0f / den;
      }
      bar();
      for (int t = threadIdx.x; t < hpg * (HD / 4); t += kThreads) {
        const int h = t / (HD / 4), d4 = (t % (HD / 4)) * 4;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int cb = 0; cb < nchunks; cb += 8) {
          f32x4 v[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            v[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (cb + jj < nchunks)
              v[jj] = *reinterpret_cast<const GAS f32x4*>(pb + ((int64_t)(cb + jj) * hpg + h) * (HD + 2) + d4);
          }
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float sc = cb + jj < nchunks ? scl[(cb + jj) * hpg + h] : 0.0f;
            acc += sc * v[jj];
          }
        }
        GAS float* dst = p.attn_o + ((int64_t)l * p.max_batch + b) * p.n_q * HD + (int64_t)(g * hpg + h) * HD + d4;
        st_pub4(dst, acc * mrow[h]);
      }
      wait_vm_all();
      bar();
      if (c.ctl) ctl_signal(c, layer_ctr(p, l, p.ctr.comb + g));
    }
  }
  return true;
}

// ------------------------------------------------------------------ dispatch
// One non-inlined function per opcode: each gets its own register allocation, and
// nothing but the task index lives across tasks in the interpreter loop.  Arguments are
// made wave-uniform (scalar registers) on entry.
#define MKD_CASE_K(KV, CALL) \
  case KV: {                 \
    constexpr int K = KV;    \
    return CALL;             \
  }

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

#define MKD_EXEC(NAME, BODY)                                                                          \
  __device__ __forceinline__ bool NAME(KParams* kp_in, LAS char* lds_in, const CAS int32_t* d_in, int32_t task_in) { \
    KParams* kp = (KParams*)uniform_u64((uint64_t)kp_in);                                             \
    const CAS int32_t* d = (const CAS int32_t*)uniform_u64((uint64_t)d_in);                           \
    LAS char* lds = (LAS char*)(uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_in); \
    const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);                            \
    Ctx c{kp, Smem(lds), d, __builtin_amdgcn_readfirstlane(task_in), wave, (int32_t)(threadIdx.x & 63), \
          wave - 1, wave == 0};                                                                       \
    BODY                                                                                              \
  }

MKD_EXEC(exec_embed, return op_embed(c);)
MKD_EXEC(exec_qkv, switch (kp->hidden) { MKD_CASE_K(256, op_qkv<K>(c)) MKD_CASE_K(2048, op_qkv<K>(c)) } return false;)
MKD_EXEC(exec_router, switch (kp->hidden) { MKD_CASE_K(256, op_rows_on_x<K>(c, false)) MKD_CASE_K(2048, op_rows_on_x<K>(c, false)) } return false;)
MKD_EXEC(exec_lm_head, switch (kp->hidden) { MKD_CASE_K(256, op_rows_on_x<K>(c, true)) MKD_CASE_K(2048, op_rows_on_x<K>(c, true)) } return false;)
MKD_EXEC(exec_oproj, switch (kp->n_q * kp->head_dim / kp->n_kv) { MKD_CASE_K(256, op_oproj<K>(c)) MKD_CASE_K(1024, op_oproj<K>(c)) } return false;)
MKD_EXEC(exec_moe_up, switch (kp->hidden) { MKD_CASE_K(256, op_moe_up<K>(c)) MKD_CASE_K(2048, op_moe_up<K>(c)) } return false;)
MKD_EXEC(exec_moe_down, switch (kp->inter) { MKD_CASE_K(128, op_moe_down<K>(c)) MKD_CASE_K(768, op_moe_down<K>(c)) } return false;)
MKD_EXEC(exec_attn, if (kp->head_dim == 128) return op_attn<128>(c); if (kp->head_dim == 64) return op_attn<64>(c); return false;)

__device__ __forceinline__ bool run_task(KParams* kp, LAS char* lds, const CAS int32_t* d, int32_t task) {
  switch (d[D_OPCODE]) {
    case OP_EMBED: return exec_embed(kp, lds, d, task);
    case OP_QKV: return exec_qkv(kp, lds, d, task);
    case OP_ROUTER: return exec_router(kp, lds, d, task);
    case OP_LM_HEAD: return exec_lm_head(kp, lds, d, task);
    case OP_OPROJ: return exec_oproj(kp, lds, d, task);
    case OP_MOE_UP: return exec_moe_up(kp, lds, d, task);
    case OP_MOE_DOWN: return exec_moe_down(kp, lds, d, task);
    case OP_ATTN: return exec_attn(kp, lds, d, task);
    default: return true;
  }
}

// Trace record of a finished task (controller lane 0; fields in LDS were set by the task).
__device__ __forceinline__ void trace_task(KParams* kp, LAS int32_t* mi, const CAS int32_t* d, uint64_t t0) {
  GAS uint64_t* trace = gas(kp->trace);
  if (trace && threadIdx.x == 0) {
    const int32_t gi = d[D_GIDX];
    if (gi >= 0 && gi < kp->trace_cap) {
      const uint64_t ready = ((uint64_t)(uint32_t)mi[MI_READY_HI] << 32) | (uint32_t)mi[MI_READY_LO];
      GAS uint64_t* r = trace + (int64_t)gi * 4;
      const uint64_t tend = wall_clock64();
      r[0] = t0;
      r[1] = ready ? ready : t0;
      r[2] = tend;
      // meta: opcode (8 bits) | workgroup (12) | items (12) | staged - start (16, 10 ns) | done - start (16)
      const uint32_t st = mi[MI_T_STAGED] ? (uint32_t)mi[MI_T_STAGED] - (uint32_t)t0 : 0u;
      const uint32_t dn = mi[MI_T_DONE] ? (uint32_t)mi[MI_T_DONE] - (uint32_t)t0 : 0u;
      r[3] = (uint64_t)((uint32_t)d[D_OPCODE] & 0xFFu) | ((uint64_t)(blockIdx.x & 0xFFFu) << 8) |
             ((uint64_t)((uint32_t)mi[MI_ITEMS] & 0xFFFu) << 20) | ((uint64_t)min(st, 0xFFFFu) << 32) |
             ((uint64_t)min(dn, 0xFFFFu) << 48);
    }
  }
}

// Controller-owned per-task state (no other wave reads it, so no barrier is needed).
__device__ __forceinline__ void reset_task_state(LAS int32_t* mi, bool first) {
  if (threadIdx.x == 0) {
    if (first) {
      mi[MI_WAIT_CTR] = -1;
      mi[MI_WAIT_TGT] = 0;
      mi[MI_XS_LAYER] = -1;
    }
    mi[MI_ITEMS] = 0;
    mi[MI_READY_LO] = 0;
    mi[MI_READY_HI] = 0;
    mi[MI_T_STAGED] = 0;
    mi[MI_T_DONE] = 0;
  }
}

// Persistent interpreter: workgroup i walks task list i.  All waves call every task; the
// tasks' own barriers keep controller and workers in step.
__global__ void __launch_bounds__(kThreads, 1) mk_persistent(Params prm) {
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  LAS char* lds = (LAS char*)lds_raw;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  LAS int32_t* mi = reinterpret_cast<LAS int32_t*>(lds + kLdsMisc);
  const CAS int32_t* offs = cas(prm.cu_offsets);
  const int begin = offs[blockIdx.x], end = offs[blockIdx.x + 1];
  for (int t = begin; t < end; ++t) {
    // Opaque per task: argument fields are re-read (scalar cache) inside each task instead
    // of being hoisted out of the loop and kept live across every opcode body.
    uint64_t kpv = (uint64_t)kp;
    asm volatile("" : "+s"(kpv));
    KParams* kpt = (KParams*)kpv;
    const CAS int32_t* d = cas(kpt->tasks) + (int64_t)t * D_WORDS;
    reset_task_state(mi, t == begin);
    const uint64_t t0 = kpt->trace ? wall_clock64() : 0;
    const bool ok = run_task(kpt, lds, d, t);
    trace_task(kpt, mi, d, t0);
    if (!ok) break;
  }
}

// Ablation: one launch per wave of tasks; block i runs task first + i.
__global__ void __launch_bounds__(kThreads, 1) mk_wave(Params prm, int32_t first) {
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  LAS char* lds = (LAS char*)lds_raw;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  LAS int32_t* mi = reinterpret_cast<LAS int32_t*>(lds + kLdsMisc);
  const int32_t t = first + (int32_t)blockIdx.x;
  const CAS int32_t* d = cas(prm.tasks) + (int64_t)t * D_WORDS;
  reset_task_state(mi, true);
  const uint64_t t0 = prm.trace ? wall_clock64() : 0;
  run_task(kp, lds, d, t);
  trace_task(kp, mi, d, t0);
}

__global__ void mk_clear(uint32_t* counters, int32_t n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) counters[i] = 0u;
}

}  // namespace mkd

// ------------------------------------------------------------------ launch wrappers
namespace mkd {

hipError_t launch_clear(uint32_t* counters, int32_t n, hipStream_t s) {
  hipLaunchKernelGGL(mk_clear, dim3(64), dim3(256), 0, s, counters, n);
  return hipGetLastError();
}

hipError_t launch_persistent(const Params& p, int n_wg, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&mk_persistent), dim3(n_wg), dim3(kThreads),
                                    args, 0, s);
}

hipError_t launch_wave(const Params& p, int32_t first, int32_t count, hipStream_t s) {
  hipLaunchKernelGGL(mk_wave, dim3(count), dim3(kThreads), 0, s, p, first);
  return hipGetLastError();
}

int threads_per_wg() { return kThreads; }

}  // namespace mkd
