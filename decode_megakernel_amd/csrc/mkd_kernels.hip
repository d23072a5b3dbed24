// mkd_kernels.hip - the decode megakernel for gfx950: tile bodies of every opcode and
// the persistent task interpreter (plus the op-per-kernel ablation launcher).
//
// Method: "Inside the megakernel serving engine for North Mini Code" (Cohere).
//  - "What is a Megakernel?": one workgroup per compute unit, resident for the whole
//    step, walking a host-built task list in global memory; dependencies are counters
//    that producers increment and consumers spin on.
//  - "The threadblock shape": every opcode runs under one fixed shape with fixed
//    roles.  Here: 8 wave64s per workgroup walking one task list; the first wave is the
//    controller (polls of tagged data, queue claims, activation staging into LDS,
//    epilogue stores) and the other seven are workers that stream weights / K-V from
//    HBM and compute.  On gfx9 the vector-memory counter is in order and shared by
//    loads, stores and atomics, so a wave with weight loads in flight cannot get a quick
//    answer from a poll, a small load or a store; keeping every latency-critical access
//    on a wave that never streams weights is what lets the workers keep HBM busy while
//    the controller resolves dependencies.  Barriers only order LDS, so worker loads
//    stay in flight across them.
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

#include <algorithm>

#include "mkd_common.h"
#include "mkd_device.h"

namespace mkd {

// ------------------------------------------------------------------ LDS layout
// One workgroup per CU is forced by the LDS footprint (> half of the 160 KB).  Regions:
// activation staging / attention pages and merge (xs: 144 KB, 16 tokens x 2048 fp32 plus
// room for the attention pages held in LDS), per-row results of a tile (rowsum), routing
// tables (route) and controller state (misc).
constexpr int kLdsRowsumBytes = 8192;
constexpr int kLdsRouteBytes = 6400;
constexpr int kLdsMiscBytes = 1024;
constexpr int kXsBytes = 147456;
constexpr int kLdsBytes = kXsBytes + kLdsRowsumBytes + kLdsRouteBytes + kLdsMiscBytes;
#ifndef MKD_MAXP
#define MKD_MAXP 1
#endif
constexpr int kMaxPagesPerWave = MKD_MAXP;  // attention pages each worker holds in registers
#ifndef MKD_LDS_PAGES
#define MKD_LDS_PAGES 4
#endif
constexpr int kMaxLdsPages = MKD_LDS_PAGES;  // attention pages each worker prefetches into LDS
#ifndef MKD_MACC
#define MKD_MACC 1536
#endif
constexpr int kMaccOffset = MKD_MACC;  // output-task accumulators, floats after rowsum
#ifndef MKD_RING
#define MKD_RING 8
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
  __device__ explicit Smem(LAS char* base) {
    const int xb = kXsBytes;
    xs = reinterpret_cast<LAS float*>(base);
    rowsum = reinterpret_cast<LAS float*>(base + xb);
    route = reinterpret_cast<LAS int32_t*>(base + xb + kLdsRowsumBytes);
    mi = reinterpret_cast<LAS int32_t*>(base + xb + kLdsRowsumBytes + kLdsRouteBytes);
    mf = reinterpret_cast<LAS float*>(base + xb + kLdsRowsumBytes + kLdsRouteBytes + 768);
  }
};
// misc int slots
constexpr int MI_OK = 1;         // controller -> workers: inputs ready (0: abort)
constexpr int MI_ITEMS = 4;      // trace: items claimed by the current task
constexpr int MI_READY_LO = 6;   // trace: when the current task's first wait completed
constexpr int MI_READY_HI = 7;
constexpr int MI_XS_LAYER = 8;   // layer whose normed input xs holds (-1: none)
constexpr int MI_ROUTE_LAYER = 9;  // layer whose routing tables the route area holds (-1: none)
constexpr int MI_WFAIL = 10;     // a worker's wait on tagged data gave up (the step is aborted)
constexpr int MI_NEXT = 16;      // [2][2] claimed items (ping-pong): (item, task index) pairs
constexpr int MI_T_STAGED = 14;  // trace: low 32 bits of the clock when inputs were staged
constexpr int MI_T_DONE = 15;    // trace: low 32 bits of the clock when the workers finished
constexpr int MI_TOK = 32;       // [16] token list of the current GEMV

// Routing table offsets inside Smem::route (int32 units; at most B*k <= 256 entries
// and min(E, B*k) <= 256 active experts).
constexpr int RT_IDS = 0;       // [16][16] selected experts per token
constexpr int RT_W = 256;       // [16][16] routing weights (float bits)
constexpr int RT_NACT = 512;    // number of active experts
constexpr int RT_ACT = 520;     // [256] active experts, ascending
constexpr int RT_OFF = 776;     // [257] CSR offsets of each active expert's (token, slot) list
constexpr int RT_FLAT = 1036;   // [256] b*k + j entries, experts ascending, tokens ascending
constexpr int RT_EPOS = 1292;   // [256] entry b*k + j: (active expert index << 16) | position in its list
constexpr int kRouteWords = kRouteTableWords;  // the whole table, as published (tagged) by the route builder
static_assert(RT_EPOS + 256 == kRouteWords, "published table covers the routing area");
static_assert(kRouteWords * 4 <= kLdsRouteBytes, "routing tables must fit the route area");

// ------------------------------------------------------------------ task context
struct Ctx {
  KParams* kp;              // kernel arguments (constant segment)
  Smem s;
  const CAS int32_t* d;     // descriptor
  int32_t task;             // global task index
  int32_t tw, lane, wi;     // wave in the workgroup (uniform), lane, worker index (tw - 1)
  int32_t nw;               // worker waves (7)
  int32_t tid, tthreads;    // thread index in the workgroup, threads in the workgroup
  bool ctl;                 // the first wave: the controller
};

__device__ __forceinline__ GAS uint32_t* layer_ctr(const DParams& p, int l, int off) {
  return p.counters + (int64_t)l * p.ctr.per_layer + off;
}
// Cached length of sequence b as the kernel uses it: clamped to what the page-table row
// can map (0 .. max_pages * page - 1), so that no index derived from it leaves the page
// table, the attention items or their partials.  The host validates its mirror of the
// lengths; a device length outside that range is reported by the embedding task
// (check_seq_lens) and the step goes on with the clamped value.
__device__ __forceinline__ int seq_len_of(const DParams& p, int b) {
  return min(max(p.seq_lens[b], 0), p.max_pages * p.page - 1);
}

// Workgroup barrier (orders LDS; worker loads in flight stay in flight across it).
__device__ __forceinline__ void bar(const Ctx&) { __syncthreads(); }

// ------------------------------------------------------------------ controller primitives
// Claimer queues: claimer i of n takes item i first without touching the queue, then
// items n + (queue head), so the claimers' first items cost no atomic and the queue
// only sees the later claims, spread over time.  The claimer index and count are the
// descriptor's ARG0 and ARG1 (the MoE-up queue moves the static items to the claimers
// that are free first; its queue items start at `base`).
// Issue a claim without waiting for the reply: the returned item (lane 0) is only
// consumed by ctl_claim_put, placed where the reply has had time to arrive (the
// wait-counter pass waits for it there).
__device__ __forceinline__ uint32_t ctl_claim_issue(Ctx& c, GAS uint32_t* head, int32_t base) {
  uint32_t v = 0;
  if (c.lane == 0) {
    v = (uint32_t)base + ctr_add(head, 1u);
    c.s.mi[MI_ITEMS] += 1;
  }
  return v;
}
// Claim entry k (0 or 1) holds the item and the index of the task it belongs to, written
// and read as one 64-bit LDS word.  A claimer loop ends when every wave reads an item
// past the end of the queue; the controller may read it first and start its next task,
// whose first claim overwrites entry 0 before a slower worker has read it.  The task
// tag makes such an entry read as the end of the queue, which is right: the controller
// only moves on after reading this task's end.
__device__ __forceinline__ void ctl_claim_put(Ctx& c, int k, uint32_t v) {
  if (c.lane == 0) *reinterpret_cast<LAS u32x2*>(c.s.mi + MI_NEXT + 2 * k) = u32x2{v, (uint32_t)c.task};
}
__device__ __forceinline__ int32_t read_claim(Ctx& c, int k) {
  const u32x2 e = *reinterpret_cast<const LAS u32x2*>(c.s.mi + MI_NEXT + 2 * k);
  const uint32_t item = __builtin_amdgcn_readfirstlane(e.x), tag = __builtin_amdgcn_readfirstlane(e.y);
  return tag == (uint32_t)c.task ? (int32_t)item : 0x7FFFFFFF;
}

__device__ __forceinline__ void ctl_set_ok(Ctx& c, bool ok) {
  if (c.lane == 0) c.s.mi[MI_OK] = ok ? 1 : 0;
}
__device__ __forceinline__ int32_t read_mi(Ctx& c, int slot) { return __builtin_amdgcn_readfirstlane(c.s.mi[slot]); }
__device__ __forceinline__ bool read_ok(Ctx& c) { return read_mi(c, MI_OK) != 0 && read_mi(c, MI_WFAIL) == 0; }

// ------------------------------------------------------------------ tagged-data waits
// Copy n tagged words into LDS, each thread of the team taking words tid, tid + tthreads,
// ... in passes of W words: src(i) is the address of word i, dst(i) where its payload
// goes.  A word whose tag is not this step's epoch is read again (after a short sleep)
// until it is; the watchdog and the abort flag bound the wait.  No barrier inside: every
// wave may call it with its share, and the caller synchronises the team.  On failure a
// worker marks MI_WFAIL, so that the team leaves the task after its next barrier.
// Words per thread per round of the team-wide waits that stage a whole layer input: the
// normed input (batch x hidden plus the row-tile sums of squares) and the combined
// attention of the O-proj.  Measured at batch 1, 4 and 16 (8K): rounds of 12 or 16 words
// for both were 1-5% slower than these widths.
#ifndef MKD_W_X
#define MKD_W_X 5
#endif
#ifndef MKD_W_A
#define MKD_W_A 8
#endif
constexpr int kStageXWords = MKD_W_X;
constexpr int kStageAWords = MKD_W_A;
#ifndef MKD_POLL_SLEEP
#define MKD_POLL_SLEEP 1
#endif
struct NoScale {
  __device__ float operator()(int) const { return 1.0f; }
};
template <int W, class Src, class Dst, class Scale = NoScale>
__device__ __forceinline__ bool team_poll(const Ctx& c, uint32_t ep, int n, Src src, Dst dst, Scale scale = Scale()) {
  const DParams p = device_view(*c.kp);
  bool ok = true;
  for (int base = 0; base < n && ok; base += W * c.tthreads) {
    uint64_t w[W];
    float sc[W];  // plain (read-only) factors, loaded together with the tagged words
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const int i = base + c.tid + u * c.tthreads;
      w[u] = i < n ? ld_tag(src(i)) : tag_word(0.0f, ep);
      sc[u] = i < n ? scale(i) : 0.0f;
    }
    int32_t spins = 0;
    while (true) {
      bool ready = true;
#pragma unroll
      for (int u = 0; u < W; ++u) ready = ready && tag_is(w[u], ep);
      if (ready) break;
      if ((++spins & 63) == 0 && aborted(p)) { ok = false; break; }
      if (spins > p.spin_limit) {
        uint32_t seen = 0;
#pragma unroll
        for (int u = 0; u < W; ++u)
          if (!tag_is(w[u], ep)) seen = (uint32_t)(w[u] >> 32);
        report_error(p, 1u, c.task, G_TAGGED, seen, ep);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(MKD_POLL_SLEEP);
#pragma unroll
      for (int u = 0; u < W; ++u) {
        const int i = base + c.tid + u * c.tthreads;
        if (!tag_is(w[u], ep)) w[u] = ld_tag(src(i));
      }
    }
    if (ok) {
#pragma unroll
      for (int u = 0; u < W; ++u) {
        const int i = base + c.tid + u * c.tthreads;
        if (i < n) {
          if constexpr (__is_same(Scale, NoScale)) dst(i) = tag_val(w[u]);
          else dst(i) = tag_val(w[u]) * sc[u];
        }
      }
    }
  }
  if (!ok && !c.ctl) c.s.mi[MI_WFAIL] = 1;
  // trace: the task's inputs are ready when its first wait on tagged data completes
  if (ok && c.ctl && c.lane == 0 && c.s.mi[MI_READY_LO] == 0 && c.s.mi[MI_READY_HI] == 0) {
    const uint64_t t = wall_clock64();
    c.s.mi[MI_READY_LO] = (int32_t)(uint32_t)t;
    c.s.mi[MI_READY_HI] = (int32_t)(uint32_t)(t >> 32);
  }
  return ok;
}

// ------------------------------------------------------------------ GEMV tile (workers)
// Weight rows of a tile: up to four segments of n1 rows each (the last may be shorter)
// with a common leading dimension, at element offsets seg0..seg3 from a wave-uniform
// base (32 bits: a tile's rows lie within a few hundred MB of its base).  With separate
// activation blocks (the output tasks: O-proj column blocks, or different experts, in the
// segments; n1 = 2^xsh), the rows of segment s multiply xs + s * xstep + tok[j] * xld, or
// with an offset table xs + (xtab[s] - xbase) * xstep + tok[j] * xld; otherwise every row
// multiplies xs + tok[j] * xld (xld = 0: the row length).  Two segments hold the two
// halves of RoPE pairs or gate|up rows.
struct RowSrc {
  const GAS uint16_t* base;
  uint32_t seg0, seg1, seg2, seg3;
  uint32_t ld;
  int32_t n1;
  int32_t xld;
  int32_t xstep, xsh;
  // segments from a table (expert ids in LDS): segment s starts at eids[s] * escale + seg0
  const LAS int32_t* eids;
  uint32_t escale;
  // activation blocks from a table (LDS), or evenly spaced when null
  const LAS int32_t* xtab;
  int32_t xbase;
  // with xtab: segment s has its own token count xtab[s + 1] - xtab[s], and its sums go to
  // rowsum[(xtab[s] - xbase + j) * n1 + row % n1] (one slot per activation row)
  int32_t segtok;
  __device__ uint32_t row_off(int i) const {
    if (eids) return (uint32_t)eids[i >> xsh] * escale + seg0 + (uint32_t)(i & (n1 - 1)) * ld;
    if (i < n1) return seg0 + (uint32_t)i * ld;
    if (i < 2 * n1) return seg1 + (uint32_t)(i - n1) * ld;
    if (i < 3 * n1) return seg2 + (uint32_t)(i - 2 * n1) * ld;
    return seg3 + (uint32_t)(i - 3 * n1) * ld;
  }
  __device__ int32_t x_off(int i) const { return ((xtab ? xtab[i >> xsh] - xbase : (i >> xsh))) * xstep; }
};
__device__ __forceinline__ RowSrc row_src(const GAS uint16_t* b1, const GAS uint16_t* b2, int64_t ld, int n1) {
  return RowSrc{b1, 0u, (uint32_t)(b2 - b1), 0u, 0u, (uint32_t)ld, n1, 0, 0, 0, nullptr, 0u, nullptr, 0, 0};
}

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
  static_assert(K % 64 == 0, "row length must be a multiple of 64");
};

// Address of chunk f of this worker's share: row step f / CPL, 16-byte chunk f % CPL.
template <int K>
__device__ __forceinline__ uint32_t gemv_chunk_off(const Ctx& c, const RowSrc& src, int f) {
  using G = Gemv<K>;
  const int si = f / G::CPL, cc = f % G::CPL;
  const int row = (c.wi + c.nw * si) * G::RPS + c.lane / G::LPR;
  const int kc = c.lane % G::LPR + G::LPR * cc;
  return src.row_off(row) + (uint32_t)kc * 8u;
}

// Worker side of a GEMV tile (includes the task's two barriers).  The worker's F chunks
// (its row steps w, w+7, ... times CPL) stream through a ring of kRing loads: the first
// kRing are issued before the first barrier (weight prefetch while the controller waits
// for the inputs), the rest as chunks are consumed.  Every ring slot issues exactly one
// load per round (slots past F load a small dummy line that stays in the cache; the
// addresses are a wave-uniform base plus a 32-bit lane offset), so the loop body is
// straight-line and the wait-counter pass keeps kRing loads in flight.
// rowsum[row * nb + j] = W[row] . x_j, x_j = xs + xo(row) + tok[j] * xld, rows < R.  NB bounds nb.
// `stage` runs between the prefetch and the first barrier: the worker's share of a
// team-wide wait on tagged inputs (a no-op when the controller stages alone).
// Staged activations in LDS: rows of K fp32 values back to back, each row split so that
// the first four values of every 8-value chunk fill its first half and the last four its
// second half.  The lane that multiplies chunk kc (16 bytes of bf16 weights) reads its
// activations as two 16-byte words at kc * 4 and K / 2 + kc * 4: neighbouring lanes read
// neighbouring 16-byte slots, so a 64-lane read touches every bank once (with the natural
// layout the 32-byte stride between lanes made every read a two-way bank conflict).
// xsplit<K>(i) is the position of element i of the row-major activation block.
template <int K>
__device__ __forceinline__ int xsplit(int i) {
  const int r = i / K, k = i - r * K;
  return r * K + ((k & 4) ? K / 2 : 0) + ((k >> 3) << 2) + (k & 3);
}
template <int K>
__device__ __forceinline__ float dot8x(const u32x4 w, const LAS float* row, int kc) {
  const LAS f32x4* lo = reinterpret_cast<const LAS f32x4*>(row + kc * 4);
  const LAS f32x4* hi = reinterpret_cast<const LAS f32x4*>(row + K / 2 + kc * 4);
  return dot8(w, lo[0], hi[0]);
}

struct NoStage {
  __device__ bool operator()() const { return true; }
};
template <int K, int NB, bool XSEG, class Stage>
__device__ __forceinline__ bool gemv_tile(const Ctx& c, const RowSrc& src, int R, const LAS float* xs,
                                          const LAS int32_t* tok, int nb, LAS float* rowsum, Stage stage) {
  using G = Gemv<K>;
  const int S = (R + G::RPS - 1) / G::RPS;
  const int ns = c.wi < S ? (S - c.wi + c.nw - 1) / c.nw : 0;
  const int F = ns * G::CPL;
  const GAS u32x4* dum = reinterpret_cast<const GAS u32x4*>(gas(c.kp->dummy)) + c.lane;
  u32x4 ring[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) ring[r] = ld_stream16(r < F ? (const GAS void*)(src.base + gemv_chunk_off<K>(c, src, r)) : (const GAS void*)dum);
  stage();
  bar(c);
  if (!read_ok(const_cast<Ctx&>(c))) return false;
  float acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = 0.0f;
  int toff[NB];  // token row offsets into xs (wave-uniform)
  const int xld = src.xld ? src.xld : K;
#pragma unroll
  for (int j = 0; j < NB; ++j) toff[j] = (NB == 1 || j < nb) ? __builtin_amdgcn_readfirstlane(tok[j]) * xld : 0;
  for (int base = 0; base < F; base += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int f = base + r;
      const u32x4 w = ring[r];
      const int fn = f + kRing;
      ring[r] = ld_stream16(fn < F ? (const GAS void*)(src.base + gemv_chunk_off<K>(c, src, fn)) : (const GAS void*)dum);
      if (f < F) {
        const int cc = f % G::CPL;
        const int kc = c.lane % G::LPR + G::LPR * cc;
        const int row = (c.wi + c.nw * (f / G::CPL)) * G::RPS + c.lane / G::LPR;
        const int xrow = XSEG ? src.x_off(row) : 0;
        // tokens of this row step (its RPS rows lie in one segment)
        int nbs = nb, ebase = 0;
        if (XSEG && src.segtok) {
          const int sg = __builtin_amdgcn_readfirstlane(row >> src.xsh);
          ebase = __builtin_amdgcn_readfirstlane(src.xtab[sg]) - src.xbase;
          nbs = __builtin_amdgcn_readfirstlane(src.xtab[sg + 1]) - src.xbase - ebase;
        }
        if (NB > 1 && nbs == 1) {
          // one token in this row step (an expert with a single token): no group of four
          acc[0] += dot8x<K>(w, xs + xrow + toff[0], kc);
        } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (NB == 1 || (j & ~3) < nbs) {
            acc[j] += dot8x<K>(w, xs + xrow + toff[j], kc);
          }
          // tokens go in groups of four without a branch inside a group, so that the
          // group's LDS reads overlap (a token past nb reads token 0's row, toff = 0, and
          // its sum is never stored); the barrier bounds the activations in flight to one
          // group (32 registers)
          if (NB > 1 && (j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        }
        if (cc == G::CPL - 1) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if (NB == 1 || j < nbs) {
              const float t = group_sum<G::LPR>(acc[j]);
              const int slot = XSEG && src.segtok ? (ebase + j) * src.n1 + (row & (src.n1 - 1)) : row * nb + j;
              if (c.lane % G::LPR == 0 && row < R) rowsum[slot] = t;
            }
            acc[j] = 0.0f;
          }
        }
      }
    }
  }
  bar(c);
  return true;
}

// Worker side of a GEMV tile whose weights fit in LDS beside the staged input (QKV tiles at
// small batch): every chunk of the worker's share is copied into its LDS region before the
// input is waited for (the copies complete before the first barrier), then the tile is
// computed from LDS.  The region of worker w starts after the chunks of workers 0 .. w-1.
template <int K, int NB, class Stage>
__device__ __forceinline__ bool gemv_tile_lds(const Ctx& c, const RowSrc& src, int R, const LAS float* xs,
                                              const LAS int32_t* tok, int nb, LAS float* rowsum, Stage stage,
                                              LAS char* region) {
  using G = Gemv<K>;
  const int S = (R + G::RPS - 1) / G::RPS;
  const int ns = c.wi < S ? (S - c.wi + c.nw - 1) / c.nw : 0;
  const int F = ns * G::CPL;
  const int before = c.wi * (S / c.nw) + min(c.wi, S % c.nw);  // row steps of workers 0 .. wi-1
  LAS char* mine = region + before * G::CPL * 1024;
  for (int f = 0; f < F; ++f) dma16(src.base + gemv_chunk_off<K>(c, src, f), mine + f * 1024);
  stage();
  bar(c);
  if (!read_ok(const_cast<Ctx&>(c))) return false;
  float acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = 0.0f;
  int toff[NB];
  const int xld = src.xld ? src.xld : K;
#pragma unroll
  for (int j = 0; j < NB; ++j) toff[j] = (NB == 1 || j < nb) ? __builtin_amdgcn_readfirstlane(tok[j]) * xld : 0;
  for (int f = 0; f < F; ++f) {
    const u32x4 w = *reinterpret_cast<const LAS u32x4*>(mine + f * 1024 + c.lane * 16);
    const int cc = f % G::CPL;
    const int kc = c.lane % G::LPR + G::LPR * cc;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (NB == 1 || j < nb) {
        acc[j] += dot8x<K>(w, xs + toff[j], kc);
      }
    }
    if (cc == G::CPL - 1) {
      const int row = (c.wi + c.nw * (f / G::CPL)) * G::RPS + c.lane / G::LPR;
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
  bar(c);
  return true;
}

// XSEG: the segments of the tile read different activation blocks (output tasks).
template <int K, bool XSEG = false, class Stage = NoStage>
__device__ __forceinline__ bool worker_gemv(const Ctx& c, const RowSrc& src, int R, const LAS float* xs,
                                            const LAS int32_t* tok, int nb, LAS float* rowsum,
                                            Stage stage = Stage()) {
  if (nb == 1) return gemv_tile<K, 1, XSEG>(c, src, R, xs, tok, nb, rowsum, stage);
  if (nb <= 4) return gemv_tile<K, 4, XSEG>(c, src, R, xs, tok, nb, rowsum, stage);
  return gemv_tile<K, kMaxBatch, XSEG>(c, src, R, xs, tok, nb, rowsum, stage);
}

// Controller side of the same two barriers.  While the workers compute, a pending claim
// reply (next_entry >= 0) is stored to its claim entry and a deferred arrive (the
// previous item's results, already stored) is completed on `flush`.
struct NoHook {
  __device__ void operator()() const {}
};
template <class Hook = NoHook>
__device__ __forceinline__ bool ctl_gemv_barriers(Ctx& c, bool ok, int next_entry = -1, uint32_t claim = 0,
                                                  Hook after_first = Hook()) {
  ctl_set_ok(c, ok);
  if (c.lane == 0 && c.s.mi[MI_T_STAGED] == 0) c.s.mi[MI_T_STAGED] = (int32_t)(uint32_t)wall_clock64();
  bar(c);
  if (!read_ok(c)) return false;
  after_first();
  if (next_entry >= 0) ctl_claim_put(c, next_entry, claim);
  bar(c);
  if (c.lane == 0 && c.s.mi[MI_T_DONE] == 0) c.s.mi[MI_T_DONE] = (int32_t)(uint32_t)wall_clock64();
  return true;
}

// ------------------------------------------------------------------ activation staging (team)
// xs[b][k] = h_l[b][k] * gamma_l[k] for every token of the batch (rows in the split layout
// of xsplit), and mf[b] = inv_rms_b:
// the RMSNorm that every consumer of layer l's input applies, with the per-token scale
// moved to the consumer's epilogue (row sums times mf[token]).  Every wave of the team
// waits for its share of the tagged residual rows and of the per-row-tile sums of squares
// (staged behind x, at xs + B * H) and writes x; after the task's first barrier the
// controller reduces the sums of squares into mf (stage_x_finish).  The staged vector is
// kept while the next tasks on this CU read the same layer's input (MI_XS_LAYER, set by
// the controller after that barrier, so that every wave of this task saw the old value).
// Returns false on abort / watchdog; `fresh` tells whether this call staged.
template <int K>
__device__ __forceinline__ bool team_stage_x(const Ctx& c, int l, bool& fresh) {
  fresh = read_mi(const_cast<Ctx&>(c), MI_XS_LAYER) != l;
  if (!fresh) return true;
  const DParams p = device_view(*c.kp);
  const int B = p.batch, H = p.hidden, NRT = p.shape.n_rt, nh = B * H;  // NRT <= 256
  const GAS uint64_t* hb = p.h + (int64_t)l * p.max_batch * H;
  const GAS uint64_t* sb = p.ss + (int64_t)l * p.max_batch * NRT;
  const GAS uint16_t* gamma = p.norm + (int64_t)l * H;
  LAS float* xs = c.s.xs;
  return team_poll<kStageXWords>(
      c, layer_tag(p.epoch, l), nh + B * NRT, [&](int i) { return i < nh ? hb + i : sb + (i - nh); },
      [&](int i) -> LAS float& { return xs[i < nh ? xsplit<K>(i) : i]; },
      [&](int i) { return i < nh ? bf16_to_f32(gamma[i % H]) : 1.0f; });
}
__device__ __forceinline__ void stage_x_finish(Ctx& c, int l, bool fresh) {
  if (!fresh) return;
  const DParams p = device_view(*c.kp);
  const int B = p.batch, H = p.hidden, NRT = p.shape.n_rt;
  const LAS float* ssx = c.s.xs + B * H;
  for (int b = 0; b < B; ++b) {
    float t = 0.0f;
    for (int r = c.lane; r < NRT; r += 64) t += ssx[b * NRT + r];
    t = group_sum<64>(t);
    if (c.lane == 0) c.s.mf[b] = 1.0f / sqrtf(t / (float)H + p.rms_eps);
  }
  if (c.lane == 0) c.s.mi[MI_XS_LAYER] = l;
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
    st_tag(p.h + (int64_t)b * H + r, v, layer_tag(p.epoch, 0));
    red[i] = v * v;
  }
  for (int b = 0; b < B; ++b) {
    float t = 0.0f;
    for (int r = c.lane; r < R; r += 64) t += red[b * R + r];
    t = group_sum<64>(t);
    if (c.lane == 0) st_tag(p.ss + (int64_t)b * p.shape.n_rt + rt, t, layer_tag(p.epoch, 0));
  }
  if (rt == 0) {
    // device lengths outside what the page-table row maps are reported (and clamped)
    if (c.lane < B && p.seq_lens[c.lane] != seq_len_of(p, c.lane))
      report_error(p, 2u, c.task, -1, (uint32_t)p.seq_lens[c.lane], (uint32_t)(p.max_pages * p.page));
    const int half = p.head_dim / 2;
    for (int i = c.lane; i < B * half; i += 64) {
      const int b = i / half, k = i % half;
      const double ang = (double)seq_len_of(p, b) * p.inv_freq[k];
      st_tag(p.rope + 2 * i, (float)cos(ang), layer_tag(p.epoch, 0));
      st_tag(p.rope + 2 * i + 1, (float)sin(ang), layer_tag(p.epoch, 0));
    }
  }
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
  const RowSrc src = row_src(wl + ((int64_t)hh * hd + j0) * H, wl + ((int64_t)hh * hd + half + j0) * H, H, PB);
  bool fresh = false;
  auto stage = [&]() { return team_stage_x<K>(c, l, fresh); };
  if (!c.ctl) {
    // the whole tile in LDS after the staged input and its sums of squares, when it fits
    const int xs_floats = kXsBytes / 4;
    const int used = B * H + B * p.shape.n_rt;
    if (B == 1 && used + 2 * PB * K / 2 <= xs_floats)
      return gemv_tile_lds<K, 1>(c, src, 2 * PB, c.s.xs, c.s.mi + MI_TOK, B, c.s.rowsum, stage,
                                 reinterpret_cast<LAS char*>(c.s.xs + used));
    return worker_gemv<K>(c, src, 2 * PB, c.s.xs, c.s.mi + MI_TOK, B, c.s.rowsum, stage);
  } else {
    const bool rope_head = hh < p.n_q + p.n_kv;
    // the epilogue's first (cos, sin) pair per lane (tagged by the embedding task) is read
    // before the staging, so that it arrives while the workers compute
    uint64_t cw0 = 0, sw0 = 0;
    const GAS uint64_t* rope0 = p.rope + ((int64_t)(c.lane % B) * half + j0 + c.lane / B) * 2;
    if (rope_head && c.lane < PB * B) {
      cw0 = ld_tag(rope0);
      sw0 = ld_tag(rope0 + 1);
    }
    const bool ok = stage();
    if (ok && c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
    if (!ctl_gemv_barriers(c, ok, -1, 0, [&]() { stage_x_finish(c, l, fresh); })) return false;
    const uint32_t ep0 = layer_tag(p.epoch, 0);
    for (int i = c.lane; i < PB * B; i += 64) {
      const int r = i / B, b = i % B, dim = j0 + r;
      const float a = c.s.rowsum[r * B + b] * c.s.mf[b], bb = c.s.rowsum[(PB + r) * B + b] * c.s.mf[b];
      const int pos = seq_len_of(p, b);
      float o1 = a, o2 = bb;
      if (rope_head) {
        const GAS uint64_t* rp = p.rope + ((int64_t)b * half + dim) * 2;
        uint64_t cw = i == c.lane ? cw0 : ld_tag(rp), sw = i == c.lane ? sw0 : ld_tag(rp + 1);
        int32_t spins = 0;
        while (!tag_is(cw, ep0) || !tag_is(sw, ep0)) {  // written long before (embedding task)
          if ((++spins & 63) == 0 && aborted(p)) break;
          if (spins > p.spin_limit) {
            report_error(p, 1u, c.task, G_TAGGED, (uint32_t)(cw >> 32), ep0);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          cw = ld_tag(rp);
          sw = ld_tag(rp + 1);
        }
        const float cs = tag_val(cw), sn = tag_val(sw);
        o1 = a * cs - bb * sn;
        o2 = bb * cs + a * sn;
      }
      if (hh < p.n_q) {
        GAS uint64_t* q = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * hd + (int64_t)hh * hd;
        st_tag(q + dim, o1, layer_tag(p.epoch, l));
        st_tag(q + dim + half, o2, layer_tag(p.epoch, l));
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
    // queries leave as tagged words; a K or V tile raises its flag once its pool stores
    // have completed, so that the attention item holding the new token's page may read it
    if (hh >= p.n_q && c.lane == 0) {
      wait_vm_all();
      st_tag(p.kvflag + ((int64_t)l * 2 * p.n_kv + (hh - p.n_q)) * 64 + c.d[D_ARG3], 1.0f, layer_tag(p.epoch, l));
    }
  }
  return true;
}

__device__ __forceinline__ bool route_build(Ctx& c, int l);

// ------------------------------------------------------------------ OP_ROUTER / OP_LM_HEAD
// Plain GEMV tiles on the normed input: router logits (layer l) or vocabulary logits
// (final norm, tied embedding).
template <int K>
__device__ __forceinline__ bool op_rows_on_x(Ctx& c, bool lm_head) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], r0 = c.d[D_ARG0], R = c.d[D_ARG1];
  const int H = p.hidden, B = p.batch;
  const GAS uint16_t* base = lm_head ? p.embed + (int64_t)r0 * H : p.w_router + ((int64_t)l * p.n_experts + r0) * H;
  const RowSrc src = row_src(base, base, H, R);
  bool fresh = false;
  auto stage = [&]() { return team_stage_x<K>(c, l, fresh); };
  if (!c.ctl) {
    if (!worker_gemv<K>(c, src, R, c.s.xs, c.s.mi + MI_TOK, B, c.s.rowsum, stage)) return false;
  } else {
    const bool ok = stage();
    if (ok && c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
    if (!ctl_gemv_barriers(c, ok, -1, 0, [&]() { stage_x_finish(c, l, fresh); })) return false;
    for (int i = c.lane; i < R * B; i += 64) {
      const int r = i / B, b = i % B;
      const float v = c.s.rowsum[i] * c.s.mf[b];
      if (lm_head) st_pub(p.logits + (int64_t)b * p.vocab + r0 + r, v);
      else st_tag(p.router + ((int64_t)l * p.max_batch + b) * p.n_experts + r0 + r, v, layer_tag(p.epoch, l));
    }
  }
  // the layer's route builder (first router tile): routing tables for everyone
  if (!lm_head && c.d[D_ARG2] == 1) return route_build(c, l);
  return true;
}

// ------------------------------------------------------------------ routing
// ROUTER_TOPK + ROUTE_FINALIZE + MOE_GATHER in LDS: top-k of each token's router logits
// (descending, ties to the lower expert index), softmax over the selected logits, then
// the active experts in ascending order and, per expert, its (token, slot) entries in
// ascending token order.  The tables stay valid for the rest of the layer (the output
// task after the MoE-up claimer on the same CU reuses them).
//
// Top-k of token b by one wave: k rounds of a wave argmax, each a DPP maximum of the
// lanes' best remaining logits and a DPP minimum of the expert indices that reach it
// (ties go to the lower index); lane 0 writes the ids and the softmax weights.
// Router logits of token b (lane e holds experts e, e + 64, ...), waited for on their tags.
// With `once`, a single read: returns false unless every logit is already there.
// Otherwise the read repeats until they are (false on abort or watchdog).
__device__ __forceinline__ bool route_load(const Ctx& c, const DParams& p, int l, int b, float (&v)[4],
                                           bool once = false) {
  const int E = p.n_experts;  // E <= 256
  const uint32_t ep = layer_tag(p.epoch, l);
  const GAS uint64_t* r = p.router + ((int64_t)l * p.max_batch + b) * E;
  uint64_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = c.lane + 64 * i;
    w[i] = e < E ? ld_tag(r + e) : tag_word(-INFINITY, ep);
  }
  int32_t spins = 0;
  while (true) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) ready = ready && tag_is(w[i], ep);
    const uint64_t pending = __ballot(!ready);
    if (pending == 0) break;
    if (once) return false;
    if ((++spins & 63) == 0 && aborted(p)) return false;
    if (spins > p.spin_limit) {
      if (c.lane == __builtin_ctzll(pending)) report_error(p, 1u, c.task, G_TAGGED, (uint32_t)(w[0] >> 32), ep);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = c.lane + 64 * i;
      if (!tag_is(w[i], ep)) w[i] = ld_tag(r + e);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = tag_val(w[i]);
  return true;
}
__device__ __forceinline__ void route_select(const Ctx& c, const DParams& p, int b, float (&v)[4]) {
  const int E = p.n_experts, k = p.top_k;  // k <= 16
  LAS int32_t* rt = c.s.route;
  LAS float* rw = reinterpret_cast<LAS float*>(rt + RT_W);
  const int lane = c.lane;
  // round j leaves the j-th choice (logit, expert) in lane j's registers
  float myv = -INFINITY;
  int myid = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
    const float M = wave_max(bv);
    const int BI = wave_min_i(bv == M ? bi : 0x7FFFFFFF);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == BI) v[i] = -INFINITY;
    if (lane == j) {
      myv = M;
      myid = BI;
    }
  }
  // softmax over the k selected logits (lane j: choice j), the first choice being the max
  const float v0 = lane_f(myv, 0);
  const float ex = lane < k ? expf(myv - v0) : 0.0f;
  const float sum = group_sum<16>(ex);  // lanes 0..15 hold the k choices
  if (lane < k) {
    rt[RT_IDS + b * 16 + lane] = myid;
    rw[b * 16 + lane] = ex / sum;
  }
}

// Active experts (ascending) with their CSR offsets into the flat (token, slot) list, by
// one wave: lane = expert of a 64-expert block; each lane counts its entries from the
// entries' expert ids held in registers (read once, broadcast with readlane), and ballots
// give each active expert its rank and the exclusive prefix of the entry counts (counts
// <= 16: five bit planes).
__device__ __forceinline__ void route_csr(const Ctx& c, const DParams& p) {
  const int B = p.batch, E = p.n_experts, k = p.top_k, n = B * k;  // n <= 256
  LAS int32_t* rt = c.s.route;
  const int lane = c.lane;
  if (B == 1) {
    // One token: its k choices are normally k distinct experts, so the active experts are
    // the choices in ascending order, each with one entry (its choice index j); the rank
    // of choice j is the number of choices with a lower expert id.  Repeated or invalid
    // ids (only possible with NaN logits) take the general path below, which leaves such
    // entries out.
    const int id = lane < k ? rt[RT_IDS + lane] : 0x7FFFFFFF;
    int rank = 0;
    bool odd = id < 0 || id >= E;
    for (int j = 0; j < k; ++j) {
      const int x = __builtin_amdgcn_readlane(id, j);
      rank += x < id ? 1 : 0;
      odd = odd || (x == id && j != lane);
    }
    if (__ballot(lane < k && odd) == 0) {
      if (lane < k) {
        rt[RT_ACT + rank] = id;
        rt[RT_FLAT + rank] = lane;  // entry b * k + j of token 0
        rt[RT_EPOS + lane] = rank << 16;
      }
      if (lane <= k) rt[RT_OFF + lane] = lane;
      if (lane == 0) rt[RT_NACT] = k;
      return;
    }
  }
  int ev[4];  // expert of entry lane + 64 q (entry t = b * k + j)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = lane + 64 * q;
    ev[q] = t < n ? rt[RT_IDS + (t / k) * 16 + t % k] : -1;
  }
  int n_act = 0, n_ent = 0;
  for (int blk = 0; blk < E; blk += 64) {
    const int e = blk + lane;
    int m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      for (int s = 0; s < min(64, n - 64 * q); ++s) m += __builtin_amdgcn_readlane(ev[q], s) == e ? 1 : 0;
    if (e >= E) m = 0;
    const uint64_t act = __ballot(m > 0);
    int pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
      const uint64_t plane = __ballot((m >> bit) & 1);
      pre += lanes_below(plane) << bit;
      tot += __builtin_popcountll(plane) << bit;
    }
    if (m > 0) {
      const int rank = n_act + lanes_below(act);
      int at = n_ent + pre;
      rt[RT_ACT + rank] = e;
      rt[RT_OFF + rank] = at;
      int jj = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        for (int s = 0; s < min(64, n - 64 * q); ++s)
          if (__builtin_amdgcn_readlane(ev[q], s) == e) {
            rt[RT_FLAT + at++] = 64 * q + s;  // t = b * k + j
            rt[RT_EPOS + 64 * q + s] = (rank << 16) | jj++;
          }
    }
    n_act += __builtin_popcountll(act);
    n_ent += tot;
  }
  if (lane == 0) {
    rt[RT_OFF + n_act] = n_ent;
    rt[RT_NACT] = n_act;
  }
}

// ROUTER_TOPK + ROUTE_FINALIZE + MOE_GATHER, once per layer: the task of the first router
// tile, after its own logits, waits for every token's logits (tagged), builds the tables
// in its LDS with every wave (top-k per token, then the CSR by the first wave) and
// publishes the whole table as tagged words; it also stores the routing for inspection.
// Every other CU copies the table (route_layer) instead of recomputing it, so the
// routing is done as soon as the router tiles are, off the MoE-up claimers' path.
__device__ __forceinline__ bool route_build(Ctx& c, int l) {
  const DParams p = device_view(*c.kp);
  const int B = p.batch, k = p.top_k;
  bool ok = true;
  for (int b = c.tw; b < B && ok; b += c.nw + 1) {
    float v[4];
    ok = route_load(c, p, l, b, v);
    if (ok) route_select(c, p, b, v);
  }
  if (!ok) c.s.mi[MI_WFAIL] = 1;
  bar(c);
  if (read_mi(c, MI_WFAIL) != 0) return false;
  if (c.tw == 0) route_csr(c, p);
  if (c.tid == 0) c.s.mi[MI_ROUTE_LAYER] = l;
  bar(c);
  const LAS int32_t* rt = c.s.route;
  GAS uint64_t* dst = p.route_tbl + (int64_t)l * kRouteWords;
  const uint32_t ep = layer_tag(p.epoch, l);
  for (int i = c.tid; i < kRouteWords; i += c.tthreads) st_tag(dst + i, __int_as_float(rt[i]), ep);
  if (c.tid < B * k) {
    const LAS float* rw = reinterpret_cast<const LAS float*>(rt + RT_W);
    const int b = c.tid / k, j = c.tid % k;
    st_pub(p.topk_ids + ((int64_t)l * p.max_batch + b) * k + j, rt[RT_IDS + b * 16 + j]);
    st_pub(p.topk_w + ((int64_t)l * p.max_batch + b) * k + j, rw[b * 16 + j]);
  }
  return true;
}

// The tables of layer l in this CU's LDS: kept when already there, else copied from the
// published (tagged) table by every wave.
__device__ __forceinline__ bool route_layer(Ctx& c, int l) {
  const DParams p = device_view(*c.kp);
  if (read_mi(c, MI_ROUTE_LAYER) == l) return true;
  const GAS uint64_t* src = p.route_tbl + (int64_t)l * kRouteWords;
  LAS float* rt = reinterpret_cast<LAS float*>(c.s.route);
  const bool ok = team_poll<4>(
      c, layer_tag(p.epoch, l), kRouteWords, [&](int i) { return src + i; },
      [&](int i) -> LAS float& { return rt[i]; });
  if (!ok) c.s.mi[MI_WFAIL] = 1;
  bar(c);
  if (read_mi(c, MI_WFAIL) != 0) return false;
  // published before the barrier, so that every wave of the team sees the same value at
  // the next check (a task may start right after this one without another barrier)
  if (c.tid == 0) c.s.mi[MI_ROUTE_LAYER] = l;
  bar(c);
  return true;
}

// The controller copies the published table of layer l alone, without barriers, when it
// is already complete (one read, no wait): used while the workers compute another task
// (attention), so that the MoE-up claimer that follows on this CU starts with its routing
// in place.  The workers read the tables only after a later barrier.
__device__ __forceinline__ void ctl_route_ahead(Ctx& c, int l) {
  const DParams p = device_view(*c.kp);
  if (read_mi(c, MI_ROUTE_LAYER) == l) return;
  const GAS uint64_t* src = p.route_tbl + (int64_t)l * kRouteWords;
  const uint32_t ep = layer_tag(p.epoch, l);
  LAS int32_t* rt = c.s.route;
  constexpr int PER = 8;
  for (int base = 0; base < kRouteWords; base += 64 * PER) {
    uint64_t w[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + c.lane + 64 * u;
      w[u] = i < kRouteWords ? ld_tag(src + i) : tag_word(0.0f, ep);
    }
    bool ready = true;
#pragma unroll
    for (int u = 0; u < PER; ++u) ready = ready && tag_is(w[u], ep);
    if (__ballot(!ready) != 0) return;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + c.lane + 64 * u;
      if (i < kRouteWords) rt[i] = (int32_t)(uint32_t)w[u];
    }
  }
  if (c.lane == 0) c.s.mi[MI_ROUTE_LAYER] = l;
}

// Attention items of this step: (sequence, KV group, chunk of pages_per_item pages).
// First position that layer l attends to for a sequence whose new token is at pos: the
// last attn_window positions on a local-attention layer, all positions otherwise.
__device__ __forceinline__ int attn_first_pos(const DParams& p, int l, int pos) {
  const bool local = p.attn_window > 0 && (l + 1) % p.full_every != 0;
  return local ? max(0, pos - p.attn_window + 1) : 0;
}
// Pages of sequence b that layer l reads: first .. last (the new token's page).
__device__ __forceinline__ int attn_first_page(const DParams& p, int l, int b) {
  return attn_first_pos(p, l, seq_len_of(p, b)) / p.page;
}
__device__ __forceinline__ int attn_chunks(const DParams& p, int l, int b) {
  const int ppi = p.shape.pages_per_item;
  const int npg = seq_len_of(p, b) / p.page + 1 - attn_first_page(p, l, b);
  return (npg + ppi - 1) / ppi;
}
__device__ __forceinline__ int attn_item_count(const DParams& p, int l) {
  int n = 0;
  for (int b = 0; b < p.batch; ++b) n += attn_chunks(p, l, b) * p.n_kv;
  return min(n, p.max_attn_items);
}

// ------------------------------------------------------------------ OP_MOE_UP (claimer)
// Items are (active expert, tile of up_rows activation rows); weights = up_rows gate rows
// and the matching up rows; epilogue silu(gate) * up for every token routed to the expert,
// stored as tagged words that the output tasks poll.
//
// Static streaming (when at least kMinFreeClaimers claimers have no attention item and
// each of them has at most kStaticItemsPerClaimer items, i.e. at small batch): the
// free claimers take the items round robin (free claimer f: items f, f + n_free, ...) and
// stream all of them through one ring of weight loads that runs on from one item into the
// next, so no item waits for its first loads; after each item the workers meet the
// controller at a barrier, and the controller finishes that item (SiLU, stores, arrive)
// while the workers compute the next one (rows sums double-buffered).  Claimers with an
// attention item take no MoE-up item then.  Otherwise the shared queue of the pages'
// design is drained (below).
#ifndef MKD_MIN_FREE
#define MKD_MIN_FREE 64
#endif
constexpr int kMinFreeClaimers = MKD_MIN_FREE;
#ifndef MKD_STATIC_ITEMS
#define MKD_STATIC_ITEMS 4
#endif
constexpr int kStaticItemsPerClaimer = MKD_STATIC_ITEMS;
constexpr int kRowsumHalf = 1024;  // floats: the two row-sum buffers of static streaming

template <int K, int NB>
__device__ __forceinline__ bool moe_up_static(Ctx& c, const DParams& p, int l, int fi, int n_free, int n_items) {
  using G = Gemv<K>;
  const int UR = p.shape.up_rows, NT = p.shape.n_up_tiles, I = p.inter, k = p.top_k;
  const LAS int32_t* rt = c.s.route;
  const int M = fi < n_items ? (n_items - fi + n_free - 1) / n_free : 0;
  auto item_expert = [&](int m) { return __builtin_amdgcn_readfirstlane(rt[RT_ACT + (fi + m * n_free) / NT]); };
  auto item_src = [&](int m) -> RowSrc {
    const int tile = (fi + m * n_free) % NT;
    const GAS uint16_t* base =
        p.w_gate_up + (((int64_t)l * p.n_experts + item_expert(m)) * 2 * I + (int64_t)tile * UR) * p.hidden;
    return row_src(base, base + (int64_t)I * p.hidden, p.hidden, UR);
  };
  if (!c.ctl) {
    const int R = 2 * UR;
    const int S = (R + G::RPS - 1) / G::RPS;
    const int ns = c.wi < S ? (S - c.wi + c.nw - 1) / c.nw : 0;
    const int F = ns * G::CPL;  // this worker's chunks per item
    if (F == 0) {
      for (int m = 0; m < M; ++m) bar(c);
      return true;
    }
    const int FT = M * F;
    const GAS u32x4* dum = reinterpret_cast<const GAS u32x4*>(gas(c.kp->dummy)) + c.lane;
    // next load: chunk la_f of item la_m (a dummy line past the last item)
    int la_m = 0, la_f = 0;
    RowSrc sla = item_src(0);
    auto next_addr = [&]() -> const GAS void* {
      if (la_m >= M) return (const GAS void*)dum;
      const GAS void* a = (const GAS void*)(sla.base + gemv_chunk_off<K>(c, sla, la_f));
      if (++la_f == F) {
        la_f = 0;
        if (++la_m < M) sla = item_src(la_m);
      }
      return a;
    };
    u32x4 ring[kRing];
#pragma unroll
    for (int r = 0; r < kRing; ++r) ring[r] = ld_stream16(next_addr());
    // item being computed: m, its chunk f, tokens
    int m = 0, f = 0, nb = 1;
    float acc[NB];
    int toff[NB];
    auto setup_item = [&](int mm) {
      const int a = (fi + mm * n_free) / NT;
      const int o0 = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a]);
      nb = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a + 1]) - o0;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        toff[j] = (NB == 1 || j < nb) ? __builtin_amdgcn_readfirstlane(rt[RT_FLAT + o0 + j] / k) * K : 0;
        acc[j] = 0.0f;
      }
    };
    setup_item(0);
    for (int gb = 0; gb < FT; gb += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        const int g = gb + r;
        const u32x4 w = ring[r];
        ring[r] = ld_stream16(next_addr());
        if (g < FT) {
          const int cc = f % G::CPL;
          const int kc = c.lane % G::LPR + G::LPR * cc;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if (NB == 1 || (j & ~3) < nb) {
              acc[j] += dot8x<K>(w, c.s.xs + toff[j], kc);
            }
            if (NB > 1 && (j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
          if (cc == G::CPL - 1) {
            const int row = (c.wi + c.nw * (f / G::CPL)) * G::RPS + c.lane / G::LPR;
            LAS float* rs = c.s.rowsum + (m & 1) * kRowsumHalf;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              if (NB == 1 || j < nb) {
                const float t = group_sum<G::LPR>(acc[j]);
                if (c.lane % G::LPR == 0 && row < R) rs[row * nb + j] = t;
                acc[j] = 0.0f;
              }
            }
          }
          if (++f == F) {
            // item m done on this worker: meet the controller, go on with the next item
            // (its first loads are already in flight)
            f = 0;
            bar(c);
            if (++m < M) setup_item(m);
          }
        }
      }
    }
    return true;
  } else {
    if (c.lane == 0) c.s.mi[MI_T_STAGED] = (int32_t)(uint32_t)wall_clock64();
    for (int m = 0; m < M; ++m) {
      bar(c);
      if (m == 0 && c.lane == 0) c.s.mi[MI_T_DONE] = (int32_t)(uint32_t)wall_clock64();
      const int idx = fi + m * n_free, a = idx / NT, tile = idx % NT;
      const int o0 = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a]);
      const int n_e = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a + 1]) - o0;
      const LAS float* rs = c.s.rowsum + (m & 1) * kRowsumHalf;
      for (int i = c.lane; i < UR * n_e; i += 64) {
        const int r = i / n_e, jj = i % n_e;
        const int slot = rt[RT_FLAT + o0 + jj];  // b * k + j
        const float sc = c.s.mf[slot / k];
        const float gt = rs[r * n_e + jj] * sc, u = rs[(UR + r) * n_e + jj] * sc;
        const float act = gt / (1.0f + expf(-gt)) * u;
        st_tag(p.moe_act + ((int64_t)l * p.max_batch * k + slot) * I + (int64_t)tile * UR + r, act,
               layer_tag(p.epoch, l));
      }
      if (c.lane == 0) c.s.mi[MI_ITEMS] += 1;
    }
    return true;
  }
}

// Shared-queue draining (the pages' MOE_UPGATE_ACT_DRAIN): claimer i of n takes item i
// first when it had no attention item, then items from the queue.
template <int K>
__device__ __forceinline__ bool op_moe_up(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  const int UR = p.shape.up_rows, NT = p.shape.n_up_tiles, H = p.hidden, I = p.inter, k = p.top_k;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.up_claim);
  const int n_attn = attn_item_count(p, l), ci = c.d[D_ARG0], n_cl = c.d[D_ARG1];
  // static streaming when enough claimers are free of attention and each of them has a
  // few items at most (bounded by the batch's k choices per token): otherwise the
  // attention claimers, idle after their item, share the items through the queue
  const int max_items = min(p.n_experts, p.batch * k) * NT;
  const bool stat = n_cl - n_attn >= kMinFreeClaimers && max_items <= kStaticItemsPerClaimer * (n_cl - n_attn);
  if (stat && ci < n_attn) return true;  // busy with attention: no MoE-up item
  // Queue mode: static first items go to the claimers that had no attention item in this
  // step (claimer i of both queues runs on the same CU, attention first): claimer
  // i >= n_attn takes item i - n_attn.  The others reach this task only after their
  // attention item (or its combine) and start from the queue, whose items follow the
  // static ones, so no late CU holds an item back.
  int n_static = 0;
  // the layer's normed input (normally still staged by this CU's QKV or router task)
  bool fresh = false;
  const bool staged = team_stage_x<K>(c, l, fresh);
  if (!staged && !c.ctl) c.s.mi[MI_WFAIL] = 1;
  if (c.ctl) {
    n_static = max(0, n_cl - n_attn);
    if (!stat) ctl_claim_put(c, 0, ci >= n_attn ? (uint32_t)(ci - n_attn) : ctl_claim_issue(c, head, n_static));
    ctl_set_ok(c, staged);
  }
  bar(c);
  if (!read_ok(c)) return false;
  if (c.ctl) stage_x_finish(c, l, fresh);
  if (!route_layer(c, l)) return false;
  const LAS int32_t* rt = c.s.route;
  const int n_items = __builtin_amdgcn_readfirstlane(rt[RT_NACT]) * NT;
  if (stat) {
    if (p.batch == 1) return moe_up_static<K, 1>(c, p, l, ci - n_attn, n_cl - n_attn, n_items);
    if (p.batch <= 4) return moe_up_static<K, 4>(c, p, l, ci - n_attn, n_cl - n_attn, n_items);
    return moe_up_static<K, kMaxBatch>(c, p, l, ci - n_attn, n_cl - n_attn, n_items);
  }
  for (int j = 0;; ++j) {
    const int idx = read_claim(c, j & 1);
    if (idx >= n_items) break;
    const int a = idx / NT, tile = idx % NT;
    const int e = __builtin_amdgcn_readfirstlane(rt[RT_ACT + a]);
    const int o0 = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a]);
    const int n_e = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a + 1]) - o0;
    const GAS uint16_t* base = p.w_gate_up + (((int64_t)l * p.n_experts + e) * 2 * I + (int64_t)tile * UR) * H;
    const RowSrc src = row_src(base, base + (int64_t)I * H, H, UR);
    if (!c.ctl) {
      if (!worker_gemv<K>(c, src, 2 * UR, c.s.xs, c.s.mi + MI_TOK, n_e, c.s.rowsum)) return false;
    } else {
      if (c.lane < n_e) c.s.mi[MI_TOK + c.lane] = rt[RT_FLAT + o0 + c.lane] / k;
      const uint32_t nxt = ctl_claim_issue(c, head, n_static);
      if (!ctl_gemv_barriers(c, true, (j + 1) & 1, nxt)) return false;
      for (int i = c.lane; i < UR * n_e; i += 64) {
        const int r = i / n_e, jj = i % n_e;
        const int slot = rt[RT_FLAT + o0 + jj];  // b * k + j
        const float sc = c.s.mf[slot / k];
        const float gt = c.s.rowsum[r * n_e + jj] * sc, u = c.s.rowsum[(UR + r) * n_e + jj] * sc;
        const float act = gt / (1.0f + expf(-gt)) * u;
        st_tag(p.moe_act + ((int64_t)l * p.max_batch * k + slot) * I + (int64_t)tile * UR + r, act,
               layer_tag(p.epoch, l));
      }
      if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
    }
  }
  return true;
}

// ------------------------------------------------------------------ OP_MOE_DOWN (claimer)
// The page's MOE_DOWN_DRAIN, at batch >= kDownSplitBatch: items are (active expert a, chunk
// of down_rows output rows), claimed like the attention items (claimer i takes item i
// first, later items come from the queue).  An item waits for its expert's activation rows
// of its tokens (tagged, left by the MoE-up items), computes W_down[e][chunk rows] . act
// for each token and leaves the rows as tagged words y[slot][row], slot = b * k + j (the
// token and its choice), which the output tasks weight and sum.  Each item stages only its
// own expert's activations, where an output task that computed the down rows itself
// would stage every active expert's.  Below the threshold the output tasks compute the
// down rows themselves (one hop less) and this task does nothing.

template <int KI>
__device__ __forceinline__ bool op_moe_down(Ctx& c) {
  const DParams p = device_view(*c.kp);
  if (p.batch < kDownSplitBatch) return true;
  const int l = c.d[D_LAYER];
  const int DR = p.shape.down_rows, NC = p.shape.n_down_chunks, H = p.hidden, k = p.top_k, E = p.n_experts;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.down_claim);
  const int ci = c.d[D_ARG0], n_cl = c.d[D_ARG1];
  if (c.ctl) ctl_claim_put(c, 0, (uint32_t)ci);
  bar(c);
  if (!route_layer(c, l)) return false;
  const LAS int32_t* rt = c.s.route;
  const int n_items = __builtin_amdgcn_readfirstlane(rt[RT_NACT]) * NC;
  const uint32_t ep = layer_tag(p.epoch, l);
  const GAS uint64_t* abase = p.moe_act + (int64_t)l * p.max_batch * k * KI;
  for (int j = 0;; ++j) {
    const int idx = read_claim(c, j & 1);
    if (idx >= n_items) break;
    const int a = idx / NC, chunk = idx % NC;
    const int e = __builtin_amdgcn_readfirstlane(rt[RT_ACT + a]);
    const int o0 = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a]);
    const int n_e = __builtin_amdgcn_readfirstlane(rt[RT_OFF + a + 1]) - o0;
    const GAS uint16_t* base = p.w_down + (((int64_t)l * E + e) * H + (int64_t)chunk * DR) * KI;
    const RowSrc src = row_src(base, base, KI, DR);
    LAS float* xs = c.s.xs;
    // the expert's activation rows of its tokens (entry o0 + r at xs row r)
    auto stage = [&]() {
      return team_poll<8>(
          c, ep, n_e * KI, [&](int i) { return abase + (int64_t)rt[RT_FLAT + o0 + i / KI] * KI + i % KI; },
          [&](int i) -> LAS float& { return xs[xsplit<KI>(i)]; });
    };
    if (!c.ctl) {
      if (!worker_gemv<KI>(c, src, DR, c.s.xs, c.s.mi + MI_TOK, n_e, c.s.rowsum, stage)) return false;
    } else {
      const bool ok = stage();
      if (ok) {
        if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
        if (c.lane == 0) c.s.mi[MI_XS_LAYER] = -1;
      }
      const uint32_t nxt = ctl_claim_issue(c, head, n_cl);
      if (!ctl_gemv_barriers(c, ok, (j + 1) & 1, nxt)) return false;
      for (int i = c.lane; i < DR * n_e; i += 64) {
        const int r = i / n_e, jj = i % n_e;
        const int slot = rt[RT_FLAT + o0 + jj];  // b * k + j
        st_tag(p.moe_part + (int64_t)slot * H + (int64_t)chunk * DR + r, c.s.rowsum[r * n_e + jj], ep);
      }
    }
  }
  return true;
}

// ------------------------------------------------------------------ OP_OUT
// Residual row tile rt, rows [r0, r0 + R) with R = rt_rows:
//   a = W_o[rows] . attn_o        (all KV groups; the nq*hd columns are split into blocks of
//                                  hidden length, the segments of one GEMV, summed in order)
//   m = sum over active experts e (ascending) of w_{b,e} * W_down[e][rows] . act_{e,b}
//   h_{l+1}[rows] = h_l[rows] + a + m, and the tile's sum of squares per token.
// One task per row tile finishes the rows on its CU, so the O-proj and expert-down
// partial outputs never leave the CU and no last-arriver step is needed (section
// "Where the speedup comes from": the fused residual add + RMSNorm rejoins the two
// branches; "Tasks": MOE_COMBINE weights the expert outputs by the router scores).
// The O-proj part waits for the combined attention of every group, each expert group
// for its experts' up tiles; each GEMV's weights stream before its wait.
template <int KH, int KI>
__device__ __forceinline__ bool op_out(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], rt = c.d[D_ARG0];
  const int R = p.shape.rt_rows, r0 = rt * R, H = p.hidden, B = p.batch, k = p.top_k, E = p.n_experts;
  const int QD = p.n_q * p.head_dim, NSO = QD / KH;  // O-proj column blocks (<= 4)
  const int xs_floats = kXsBytes / 4;
  LAS float* acc_a = c.s.rowsum + kMaccOffset;  // [R][B] O-proj rows
  LAS float* acc_m = acc_a + R * kMaxBatch;     // [R][B] expert rows
  const int64_t hstride = (int64_t)p.max_batch * H;
  // this tile's residual rows of layer l (tagged), read now and checked at the end
  const uint32_t ep = layer_tag(p.epoch, l);
  uint64_t hold[2];
  auto hold_src = [&](int i) { return p.h + (int64_t)l * hstride + (int64_t)(i % B) * H + r0 + i / B; };
  if (c.ctl) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = c.lane + 64 * u;
      hold[u] = i < R * B ? ld_tag(hold_src(i)) : tag_word(0.0f, ep);
    }
    for (int i = c.lane; i < 2 * R * kMaxBatch; i += 64) acc_a[i] = 0.0f;
  }
  // routing tables of layer l (normally left in LDS by this CU's MoE-up claimer)
  if (read_mi(c, MI_ROUTE_LAYER) != l) {
    if (!route_layer(c, l)) return false;
  }
  // (1) O-proj: NSO * R rows of length KH; token groups that fit in LDS
  auto oproj = [&]() -> bool {
    RowSrc so;
    so.base = p.w_o + ((int64_t)l * H + r0) * QD;
    so.seg0 = 0u; so.seg1 = (uint32_t)KH; so.seg2 = 2u * KH; so.seg3 = 3u * KH;
    so.ld = (uint32_t)QD; so.n1 = R; so.xld = QD;
    so.xstep = KH; so.xsh = 31 - __builtin_clz(R);
    so.eids = nullptr; so.escale = 0u;
    so.xtab = nullptr; so.xbase = 0; so.segtok = 0;
    const int TG = min(kMaxBatch, xs_floats / QD);
    for (int t0 = 0; t0 < B; t0 += TG) {
      const int nb = min(TG, B - t0);
      // the combined attention of the group's tokens, waited for on its tags by every wave
      const GAS uint64_t* asrc = p.attn_o + ((int64_t)l * p.max_batch + t0) * QD;
      LAS float* xs = c.s.xs;
      auto stage = [&]() {
        return team_poll<kStageAWords>(c, layer_tag(p.epoch, l), nb * QD, [&](int i) { return asrc + i; },
                            [&](int i) -> LAS float& { return xs[xsplit<KH>(i)]; });
      };
      if (!c.ctl) {
        if (!worker_gemv<KH, true>(c, so, NSO * R, c.s.xs, c.s.mi + MI_TOK, nb, c.s.rowsum, stage)) return false;
      } else {
        const bool ok = stage();
        if (ok) {
          if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
          if (c.lane == 0) c.s.mi[MI_XS_LAYER] = -1;
        }
        if (!ctl_gemv_barriers(c, ok)) return false;
        for (int i = c.lane; i < R * nb; i += 64) {
          const int r = i / nb, j = i % nb;
          float a = 0.0f;
          for (int sg = 0; sg < NSO; ++sg) a += c.s.rowsum[(sg * R + r) * nb + j];
          acc_a[r * kMaxBatch + t0 + j] = a;
        }
      }
    }
      return true;
  };
  // (2) expert down rows: one GEMV per group of consecutive active experts whose (expert,
  // token) entries fit the LDS (one group for the whole layer up to batch 4), segment s =
  // expert a0 + s with its own token count, rows addressed through the routing table
  auto down = [&]() -> bool {
    const LAS int32_t* rtab = c.s.route;
    if (B >= kDownSplitBatch) {
      // the experts' rows of this tile per (token, choice), left by the MoE-down items:
      // word (b * k + j) * R + r, weighted by the router and summed in selection order
      const LAS float* rwt = reinterpret_cast<const LAS float*>(rtab + RT_W);
      LAS float* stg = c.s.xs;
      const bool ok = team_poll<8>(
          c, layer_tag(p.epoch, l), B * k * R,
          [&](int i) { return p.moe_part + (int64_t)(i / R) * H + r0 + i % R; },
          [&](int i) -> LAS float& { return stg[i]; });
      if (c.ctl) ctl_set_ok(c, ok);
      bar(c);
      if (!read_ok(c)) return false;
      if (c.ctl) {
        if (c.lane == 0) c.s.mi[MI_T_STAGED] = (int32_t)(uint32_t)wall_clock64();
        for (int i = c.lane; i < R * B; i += 64) {
          const int r = i / B, b = i % B;
          float a = acc_m[r * kMaxBatch + b];
          for (int j = 0; j < k; ++j) a += rwt[b * 16 + j] * stg[(b * k + j) * R + r];
          acc_m[r * kMaxBatch + b] = a;
        }
        if (c.lane == 0) c.s.mi[MI_XS_LAYER] = -1;
      }
      bar(c);
      return true;
    }
    const LAS float* rw = reinterpret_cast<const LAS float*>(rtab + RT_W);
    const int n_act = __builtin_amdgcn_readfirstlane(rtab[RT_NACT]);
    // entries per group: staged rows (three spare rows for the reads of a partial group of
    // four tokens) and row-sum slots (one per entry and row, below the accumulators)
    const int cap = min(xs_floats / KI - 4, kMaccOffset / R);
    for (int a0 = 0; a0 < n_act;) {
      const int ob0 = __builtin_amdgcn_readfirstlane(rtab[RT_OFF + a0]);
      int na = 1, nb = __builtin_amdgcn_readfirstlane(rtab[RT_OFF + a0 + 1]) - ob0;
      while (a0 + na < n_act) {
        const int o1 = __builtin_amdgcn_readfirstlane(rtab[RT_OFF + a0 + na]);
        const int o2 = __builtin_amdgcn_readfirstlane(rtab[RT_OFF + a0 + na + 1]);
        if (o2 - ob0 > cap) break;
        nb = max(nb, o2 - o1);
        ++na;
      }
      RowSrc sd;
      sd.base = p.w_down + (int64_t)l * E * H * KI;
      sd.seg0 = (uint32_t)r0 * KI; sd.seg1 = sd.seg2 = sd.seg3 = 0u;
      sd.ld = (uint32_t)KI; sd.n1 = R; sd.xld = KI;
      // activations entry-major: row (expert a0 + s, token j) at xs + (off[a0 + s] - off[a0] + j) * KI
      sd.xstep = KI; sd.xsh = 31 - __builtin_clz(R);
      sd.eids = rtab + RT_ACT + a0; sd.escale = (uint32_t)(H * KI);
      sd.xtab = rtab + RT_OFF + a0; sd.xbase = ob0; sd.segtok = 1;
      // activation rows of the group's (expert, token) entries in CSR order, waited for on
      // their tags by every wave: row r (entry ob0 + r) goes to xs + r * KI
      const int n_rows = __builtin_amdgcn_readfirstlane(rtab[RT_OFF + a0 + na]) - ob0;
      const GAS uint64_t* abase = p.moe_act + (int64_t)l * p.max_batch * k * KI;
      LAS float* xs = c.s.xs;
      auto stage = [&]() {
        return team_poll<12>(
            c, layer_tag(p.epoch, l), n_rows * KI,
            [&](int i) { return abase + (int64_t)rtab[RT_FLAT + ob0 + i / KI] * KI + i % KI; },
            [&](int i) -> LAS float& { return xs[xsplit<KI>(i)]; });
      };
      if (!c.ctl) {
        if (!worker_gemv<KI, true>(c, sd, na * R, c.s.xs, c.s.mi + MI_TOK, nb, c.s.rowsum, stage)) return false;
      } else {
        const bool ok = stage();
        // trace: an output task's "staged" time is when its first expert group's
        // activations were in LDS, its "done" time when its last GEMV finished
        if (c.lane == 0 && a0 == 0) c.s.mi[MI_T_STAGED] = (int32_t)(uint32_t)wall_clock64();
        if (ok) {
          if (c.lane < 16) c.s.mi[MI_TOK + c.lane] = c.lane;
          if (c.lane == 0) c.s.mi[MI_XS_LAYER] = -1;
        }
        if (!ctl_gemv_barriers(c, ok)) return false;
        if (c.lane == 0) c.s.mi[MI_T_DONE] = (int32_t)(uint32_t)wall_clock64();
        // router-weighted sum: lane (row, token) adds the token's choices in selection
        // order, each found through its entry record (active expert, position in the
        // expert's list), so the loads of one lane are independent of each other
        for (int i = c.lane; i < R * B; i += 64) {
          const int r = i / B, b = i % B;
          float a = acc_m[r * kMaxBatch + b];
          for (int j = 0; j < k; ++j) {
            const int ep = rtab[RT_EPOS + b * k + j], ae = ep >> 16;
            if (ae >= a0 && ae < a0 + na)
              a += rw[b * 16 + j] * c.s.rowsum[(rtab[RT_OFF + ae] - ob0 + (ep & 0xFFFF)) * R + r];
          }
          acc_m[r * kMaxBatch + b] = a;
        }
      }
      a0 += na;
    }
      return true;
  };
  // The two GEMVs in the order their inputs usually arrive: at batch 1 the experts'
  // activations (MoE-up streams beside attention on the CUs free of it) come before the
  // combined attention, so the expert rows go first; above, the claimers run attention
  // first and the O-proj goes first.
#ifndef MKD_DOWN_FIRST
#define MKD_DOWN_FIRST 1
#endif
  // (one call site each: the GEMV loops are inlined once)
  const bool down_first = MKD_DOWN_FIRST && B == 1;
  for (int part = 0; part < 2; ++part) {
    if ((part == 0) == down_first) {
      if (!down()) return false;
    } else {
      if (!oproj()) return false;
    }
  }
  // (3) h_{l+1}[rows] = h_l + a + m and the tile's sums of squares, as tagged words (the
  // next layer's consumers wait on them)
  if (c.ctl) {
    // the residual rows read at the start were written long before (previous layer's
    // output tasks, before any task of this layer could start); re-read any not yet seen
    int32_t spins = 0;
    while (__ballot(!tag_is(hold[0], ep) || !tag_is(hold[1], ep)) != 0) {
      if (++spins > p.spin_limit) {
        report_error(p, 1u, c.task, G_TAGGED, (uint32_t)(hold[0] >> 32), ep);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (!tag_is(hold[u], ep)) hold[u] = ld_tag(hold_src(c.lane + 64 * u));
    }
    const uint32_t ep1 = layer_tag(p.epoch, l + 1);
    LAS float* red = c.s.rowsum;  // [B][R] squares
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = c.lane + 64 * u;
      if (i < R * B) {
        const int r = i / B, b = i % B;
        const float v = tag_val(hold[u]) + acc_a[r * kMaxBatch + b] + acc_m[r * kMaxBatch + b];
        st_tag(p.h + (int64_t)(l + 1) * hstride + (int64_t)b * H + r0 + r, v, ep1);
        red[b * R + r] = v * v;
      }
    }
    if (c.lane < B) {
      float t = 0.0f;
      for (int r = 0; r < R; ++r) t += red[c.lane * R + r];
      st_tag(p.ss + ((int64_t)(l + 1) * p.max_batch + c.lane) * p.shape.n_rt + rt, t, ep1);
    }
  }
  // the workers wait for the controller's stores to be issued before they start polling for
  // the next layer's input (measured: their polls slowed this tail by about a microsecond)
  bar(c);
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
// tiles; only the page holding the new token is read after it.  Each item leaves its
// partial (o, m, l per head) as tagged words; after its claim loop, every claimer merges
// the chunks of the query heads assigned to it (log-sum-exp, below).
__device__ __forceinline__ void attn_map(const DParams& p, int l, int idx, int& b, int& g, int& chunk,
                                         int& nchunks, int& base_bg) {
  b = -1;
  int acc = 0;
  for (int bb = 0; bb < p.batch; ++bb) {
    const int nit = attn_chunks(p, l, bb);
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
  const int n_items = attn_item_count(p, l);
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.attn_claim);
  const int nw = c.nw;
  // The attention buffers go after this layer's staged normed input when both fit, so
  // the MoE-up claimer that follows on this CU finds the input still staged.  Each worker
  // then owns a region for the pages it prefetches into LDS (as many as fit, up to
  // kMaxLdsPages); its unnormalised outputs reuse the start of that region once its pages
  // are consumed.
  const int attn_fixed = 16 * HD + 2 * nw * 16 + 16 * (HD + 2);
  const int xs_floats = kXsBytes / 4;
  const int keep = p.batch * p.hidden + attn_fixed + nw * hpg * HD <= xs_floats ? p.batch * p.hidden : 0;
  const int page_floats = p.page * HD;  // K and V of one page, bf16
  const int n_lds = min(kMaxLdsPages, (xs_floats - keep - attn_fixed) / nw / page_floats);
  const int wstride = max(n_lds * page_floats, hpg * HD);
  LAS float* ab = c.s.xs + keep;
  LAS float* qs = ab;                                  // [hpg][HD] fp32 queries
  LAS float* mw = ab + 16 * HD;                        // [nw][16] running max per worker
  LAS float* lw = mw + nw * 16;                        // [nw][16] running sum
  LAS float* part = lw + nw * 16;                      // [hpg][HD + 2] merged partial
  LAS float* wreg = part + 16 * (HD + 2);              // [nw][wstride] pages, then [hpg][HD] outputs
  if (c.ctl) {
    ctl_claim_put(c, 0, (uint32_t)c.d[D_ARG0]);
    if (c.lane == 0 && keep == 0) c.s.mi[MI_XS_LAYER] = -1;
  }
  bar(c);
  for (int j = 0;; ++j) {
    const int idx = read_claim(c, j & 1);
    if (idx >= n_items) break;
    uint32_t nxt = 0;  // controller: claim reply for the next item
    int b, g = 0, chunk = 0, nchunks = 0, base_bg = 0;
    attn_map(p, l, idx, b, g, chunk, nchunks, base_bg);
    const int pos = seq_len_of(p, b);
    const int npg = pos / p.page + 1, last = npg - 1;
    // a local-attention layer reads from the page of its first position on, and masks
    // the positions before it on that page
    const int first = attn_first_pos(p, l, pos), fpg = first / p.page;
    const int c0 = fpg + chunk * ppi, c1 = min(npg, c0 + ppi);
    u32x4 kr[MAXP][NK];
    u32x2 vr[MAXP][NV];
    int lp[MAXP];
    int64_t kbase[MAXP], vbase[MAXP];
    // element offsets of page lpg's K and V blocks for (layer l, group g); false (and an
    // error report) for a page-table entry outside the pool
    auto page_base = [&](int lpg, int64_t& kb, int64_t& vb) -> bool {
      const int phys = lpg < p.max_pages ? p.page_table[(int64_t)b * p.max_pages + lpg] : -1;
      if (phys < 0 || phys >= p.n_pages) {
        if (c.lane == 0) report_error(p, 2u, c.task, -1, (uint32_t)phys, (uint32_t)p.n_pages);
        return false;
      }
      kb = ((((int64_t)l * 2 + 0) * p.n_pages + phys) * nkv + g) * (int64_t)p.page * HD;
      vb = ((((int64_t)l * 2 + 1) * p.n_pages + phys) * nkv + g) * (int64_t)p.page * HD;
      return true;
    };
    // K operand: lane holds token (lane & 15), dims kk*32 + (lane>>4)*8 + [0, 8);
    // V^T operand: lane holds dim dt*16 + (lane & 15), tokens (lane>>4)*4 + [0, 4)
    auto load_page = [&](u32x4 (&kq)[NK], u32x2 (&vq)[NV], int64_t kb, int64_t vb) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        kq[kk] = ld_stream16(p.kv_pool + kb + (c.lane & 15) * HD + kk * 32 + (c.lane >> 4) * 8);
#pragma unroll
      for (int dt = 0; dt < NV; ++dt)
        vq[dt] = ld_stream8(p.kv_pool + vb + (dt * 16 + (c.lane & 15)) * 16 + (c.lane >> 4) * 4);
    };
    // LDS copy of a page for slot s of this worker: K in the K operand's lane layout (1 KB
    // per 32 dims, read back conflict-free), V verbatim (dim-major, as in the pool)
    LAS char* wslot = reinterpret_cast<LAS char*>(wreg + (c.wi < 0 ? 0 : c.wi) * wstride);
    auto dma_page = [&](int s, int64_t kb, int64_t vb) {
      LAS char* dst = wslot + s * page_floats * 4;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        dma16(p.kv_pool + kb + (c.lane & 15) * HD + kk * 32 + (c.lane >> 4) * 8, dst + kk * 1024);
#pragma unroll
      for (int j = 0; j < NK; ++j) dma16(p.kv_pool + vb + j * 512 + c.lane * 8, dst + NK * 1024 + j * 1024);
    };
    // K and V tiles of group g for layer l have stored the new token's slot (their flags,
    // one per tile, are tagged); then an acquire makes the pool's new slot visible
    auto wait_kv_new = [&]() -> bool {
      const int tph = p.shape.qkv_tph;  // <= 64
      const uint32_t ep = layer_tag(p.epoch, l);
      const GAS uint64_t* fk = p.kvflag + ((int64_t)l * 2 * nkv + g) * 64;
      const GAS uint64_t* fv = p.kvflag + ((int64_t)l * 2 * nkv + nkv + g) * 64;
      uint64_t wk = c.lane < tph ? ld_tag(fk + c.lane) : tag_word(0.0f, ep);
      uint64_t wv = c.lane < tph ? ld_tag(fv + c.lane) : tag_word(0.0f, ep);
      int32_t spins = 0;
      while (__ballot(!tag_is(wk, ep) || !tag_is(wv, ep)) != 0) {
        if ((++spins & 63) == 0 && aborted(p)) return false;
        if (spins > p.spin_limit) {
          if (c.lane == 0) report_error(p, 1u, c.task, G_TAGGED, (uint32_t)(wk >> 32), ep);
          return false;
        }
        __builtin_amdgcn_s_sleep(1);
        if (!tag_is(wk, ep)) wk = ld_tag(fk + c.lane);
        if (!tag_is(wv, ep)) wv = ld_tag(fv + c.lane);
      }
      fence_acquire_agent();
      return true;
    };
    int lpl[kMaxLdsPages > 0 ? kMaxLdsPages : 1];  // pages in this worker's LDS slots (c1: none)
    if (!c.ctl) {
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        lp[i] = c0 + c.wi + nw * i;
        kbase[i] = 0;
        vbase[i] = 0;
        if (lp[i] < c1 && !page_base(lp[i], kbase[i], vbase[i])) lp[i] = c1;  // skip
        if (lp[i] < c1 && lp[i] != last) load_page(kr[i], vr[i], kbase[i], vbase[i]);
      }
      // the worker's next pages go to its LDS slots; the page holding the new token is
      // copied after the wait
#pragma unroll
      for (int s = 0; s < kMaxLdsPages; ++s) {
        lpl[s] = c1;
        if (s < n_lds) {
          const int lpg = c0 + c.wi + nw * (MAXP + s);
          int64_t kb = 0, vb = 0;
          if (lpg < c1 && page_base(lpg, kb, vb)) {
            lpl[s] = lpg;
            if (lpg != last) dma_page(s, kb, vb);
          }
        }
      }
      // The page holding the new token: the worker that has it waits for the group's K and
      // V flags (raised by the same QKV wave that stores the queries the controller is
      // waiting for), acquires and requests it, all before the first barrier.
      bool holds_last = false;
#pragma unroll
      for (int i = 0; i < MAXP; ++i) holds_last = holds_last || (lp[i] < c1 && lp[i] == last);
#pragma unroll
      for (int s = 0; s < kMaxLdsPages; ++s) holds_last = holds_last || (s < n_lds && lpl[s] == last);
      if (holds_last) {
        if (!wait_kv_new()) c.s.mi[MI_WFAIL] = 1;
#pragma unroll
        for (int i = 0; i < MAXP; ++i)
          if (lp[i] < c1 && lp[i] == last) load_page(kr[i], vr[i], kbase[i], vbase[i]);
#pragma unroll
        for (int s = 0; s < kMaxLdsPages; ++s) {
          if (s < n_lds && lpl[s] == last) {
            int64_t kb = 0, vb = 0;
            page_base(last, kb, vb);
            dma_page(s, kb, vb);
          }
        }
      }
    } else {
      // the group's queries (tagged, from the QKV tiles of its heads) go first, the claim
      // after them: the claim reply arrives during the compute
      const GAS uint64_t* qsrc = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * HD + (int64_t)g * hpg * HD;
      constexpr int QPL = 16 * HD / 64;  // words per lane for up to 16 heads
      const uint32_t ep = layer_tag(p.epoch, l);
      uint64_t qw[QPL];
#pragma unroll
      for (int u = 0; u < QPL; ++u) {
        const int i = c.lane + 64 * u;
        qw[u] = i < hpg * HD ? ld_tag(qsrc + i) : tag_word(0.0f, ep);
      }
      nxt = ctl_claim_issue(c, head, c.d[D_ARG1]);
      bool ok = true;
      int32_t spins = 0;
      while (true) {
        bool ready = true;
#pragma unroll
        for (int u = 0; u < QPL; ++u) ready = ready && tag_is(qw[u], ep);
        if (__ballot(!ready) == 0) break;
        if ((++spins & 63) == 0 && aborted(p)) { ok = false; break; }
        if (spins > p.spin_limit) {
          if (c.lane == 0) report_error(p, 1u, c.task, G_TAGGED, (uint32_t)(qw[0] >> 32), ep);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < QPL; ++u)
          if (!tag_is(qw[u], ep)) qw[u] = ld_tag(qsrc + c.lane + 64 * u);
      }
      if (ok) {
#pragma unroll
        for (int u = 0; u < QPL; ++u) {
          const int i = c.lane + 64 * u;
          if (i < hpg * HD) qs[i] = tag_val(qw[u]);
        }
        if (c.lane == 0 && c.s.mi[MI_READY_LO] == 0 && c.s.mi[MI_READY_HI] == 0) {
          const uint64_t t = wall_clock64();
          c.s.mi[MI_READY_LO] = (int32_t)(uint32_t)t;
          c.s.mi[MI_READY_HI] = (int32_t)(uint32_t)(t >> 32);
        }
      }
      ctl_set_ok(c, ok);
      // trace: "staged" = the first item's queries in LDS
      if (c.lane == 0 && c.s.mi[MI_T_STAGED] == 0) c.s.mi[MI_T_STAGED] = (int32_t)(uint32_t)wall_clock64();
    }
    bar(c);
    if (!read_ok(c)) return false;
    // the controller is idle until the merge: it copies this layer's routing tables (when
    // already published) for the tasks that follow on this CU
    if (c.ctl) ctl_route_ahead(c, l);
    if (!c.ctl) {
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
      auto do_page = [&](const u32x4 (&kq)[NK], const u32x2 (&vq)[NV], int lpg) {
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kq[kk]),
                                                      __builtin_bit_cast(bf16x8, qb[kk]), s, 0, 0, 0);
        if (lpg == last) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (lpg * p.page + (c.lane >> 4) * 4 + r > pos) s[r] = -INFINITY;
        }
        if (lpg == fpg && first > 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (lpg * p.page + (c.lane >> 4) * 4 + r < first) s[r] = -INFINITY;
        }
        // scores are <= 0 after the shift: the hardware base-2 exponential (no range
        // reduction needed; results below 2^-126 of the maximum flush to zero)
        const float pm = rows4_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        const float mn = fmaxf(m, pm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] - mn);
        const float ps = rows4_sum((pr[0] + pr[1]) + (pr[2] + pr[3]));
        lsum = lsum * alpha + ps;
        m = mn;
        const u32x2 pb2 = u32x2{cvt_bf16x2(pr[0], pr[1]), cvt_bf16x2(pr[2], pr[3])};
        const s16x4 pb = __builtin_bit_cast(s16x4, pb2);
#pragma unroll
        for (int dt = 0; dt < NV; ++dt) {
          o[dt] *= alpha;
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vq[dt]), pb, o[dt], 0, 0, 0);
        }
      };
#pragma unroll
      for (int i = 0; i < MAXP; ++i)
        if (lp[i] < c1) do_page(kr[i], vr[i], lp[i]);
      // pages in LDS: every copy this wave issued has landed after its own wait
      if (n_lds > 0) wait_vm_all();
#pragma unroll
      for (int s = 0; s < kMaxLdsPages; ++s) {
        if (s < n_lds && lpl[s] < c1) {
          const LAS char* src = wslot + s * page_floats * 4;
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) kr[0][kk] = *reinterpret_cast<const LAS u32x4*>(src + kk * 1024 + c.lane * 16);
#pragma unroll
          for (int dt = 0; dt < NV; ++dt)
            vr[0][dt] = *reinterpret_cast<const LAS u32x2*>(src + NK * 1024 +
                                                           ((dt * 16 + (c.lane & 15)) * 16 + (c.lane >> 4) * 4) * 2);
          do_page(kr[0], vr[0], lpl[s]);
        }
      }
      // further pages of this worker stream through the first page's registers
      for (int lpg = c0 + c.wi + nw * (MAXP + n_lds); lpg < c1; lpg += nw) {
        int64_t kb = 0, vb = 0;
        if (!page_base(lpg, kb, vb)) continue;
        if (lpg == last && !wait_kv_new()) c.s.mi[MI_WFAIL] = 1;
        load_page(kr[0], vr[0], kb, vb);
        do_page(kr[0], vr[0], lpg);
      }
      if (c.lane < 16) {
        mw[c.wi * 16 + c.lane] = m;
        lw[c.wi * 16 + c.lane] = lsum;
      }
      if (hq < hpg) {
        LAS float* ow = reinterpret_cast<LAS float*>(wslot);
#pragma unroll
        for (int dt = 0; dt < NV; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) ow[hq * HD + dt * 16 + (c.lane >> 4) * 4 + r] = o[dt][r];
      }
    }
    bar(c);
    // merge the workers: unnormalised o, running max M and sum L per head (all waves)
    for (int t = c.tid; t < hpg * HD; t += c.tthreads) {
      const int h = t / HD, dd = t % HD;
      float M = -INFINITY;
      for (int ww = 0; ww < nw; ++ww) M = fmaxf(M, mw[ww * 16 + h]);
      float acc = 0.0f, L = 0.0f;
      for (int ww = 0; ww < nw; ++ww) {
        const float sc = exp2f(mw[ww * 16 + h] - M);
        acc += sc * wreg[ww * wstride + h * HD + dd];
        L += sc * lw[ww * 16 + h];
      }
      part[h * (HD + 2) + dd] = acc;
      if (dd == 0) {
        part[h * (HD + 2) + HD] = M;
        part[h * (HD + 2) + HD + 1] = L;
      }
    }
    // the claim reply for the next item, stored after the merge: the workers' compute and
    // the merge give it time to arrive (the next item's index is read after the next barriers)
    if (c.ctl) ctl_claim_put(c, (j + 1) & 1, nxt);
    bar(c);
    // the item's partial (o, m, l per head) leaves as tagged words: no counter, no wait
    if (c.ctl) {
      GAS uint64_t* dst = p.attn_part + (int64_t)idx * hpg * (HD + 2);
      for (int i = c.lane; i < hpg * (HD + 2); i += 64) st_tag(dst + i, part[i], layer_tag(p.epoch, l));
      // trace: "done" = the first item's partial stored
      if (c.lane == 0 && c.s.mi[MI_T_DONE] == 0) c.s.mi[MI_T_DONE] = (int32_t)(uint32_t)wall_clock64();
    }
  }
  // Combine (ATTN_COMBINE): query head qh of sequence b is merged by claimer
  // (b * n_q + qh) mod n_claimers once it has left the queue.  Every item is claimed by
  // then, so the partials it waits for are being computed or stored.  The chunks of
  // (b, kv group) are staged in LDS in batches (their tags waited for by every wave), then
  // thread d merges dimension d over the chunks in order (online log-sum-exp, base 2);
  // the result leaves as tagged words for the output tasks.
  {
    const int n_cl = c.d[D_ARG1], ci = c.d[D_ARG0];
    const int n_duty = p.batch * p.n_q;
    LAS float* stg = wreg;
    const int CB = max(1, min(64, nw * wstride / (HD + 2)));  // chunks per staged batch
    for (int dj = ci; dj < n_duty; dj += n_cl) {
      const int b = dj / p.n_q, qh = dj % p.n_q, g = qh / hpg, h = qh % hpg;
      int base_bg = 0, nch = 0;
      for (int bb = 0; bb <= b; ++bb) {
        const int nit = attn_chunks(p, l, bb);
        if (bb == b) {
          base_bg += g * nit;
          nch = nit;
        } else {
          base_bg += nit * nkv;
        }
      }
      float M = -INFINITY, den = 0.0f, acc = 0.0f;
      for (int cb0 = 0; cb0 < nch; cb0 += CB) {
        const int ncb = min(CB, nch - cb0);
        const GAS uint64_t* src = p.attn_part + ((int64_t)(base_bg + cb0) * hpg + h) * (HD + 2);
        const int64_t cstride = (int64_t)hpg * (HD + 2);
        const bool ok = team_poll<8>(
            c, layer_tag(p.epoch, l), ncb * (HD + 2), [&](int i) { return src + (i / (HD + 2)) * cstride + i % (HD + 2); },
            [&](int i) -> LAS float& { return stg[i]; });
        if (c.ctl) ctl_set_ok(c, ok);
        bar(c);
        if (!read_ok(c)) return false;
        if (c.tid < HD) {
          for (int k = 0; k < ncb; ++k) {
            const float mk = stg[k * (HD + 2) + HD], lk = stg[k * (HD + 2) + HD + 1];
            const float mn = fmaxf(M, mk);
            const float sa = exp2f(M - mn), sb = exp2f(mk - mn);
            den = den * sa + lk * sb;
            acc = acc * sa + stg[k * (HD + 2) + c.tid] * sb;
            M = mn;
          }
        }
        bar(c);
      }
      if (c.tid < HD)
        st_tag(p.attn_o + ((int64_t)l * p.max_batch + b) * p.n_q * HD + (int64_t)qh * HD + c.tid, acc / den,
               layer_tag(p.epoch, l));
    }
  }
  return true;
}

// ------------------------------------------------------------------ dispatch
// The interpreter is compiled once per model geometry (row lengths of the GEMV tiles and
// the head dimension), so that each kernel holds only its own tile bodies: fewer code
// paths share the register allocation of the single persistent function.  Every opcode
// body is inlined; its arguments are made wave-uniform (scalar registers) on entry.
template <int HID, int INTER, int HD_>
struct Geom {
  static constexpr int kHidden = HID;   // QKV / router / MoE-up / O-proj block / LM-head row length
  static constexpr int kInter = INTER;  // expert down row length
  static constexpr int kHd = HD_;       // head dimension
};
using GeomFull = Geom<2048, 768, 128>;
using GeomTiny = Geom<256, 128, 64>;

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

#define MKD_EXEC(NAME, BODY)                                                                          \
  template <class G>                                                                                  \
  __device__ __forceinline__ bool NAME(KParams* kp_in, LAS char* lds_in, const CAS int32_t* d_in, int32_t task_in) { \
    KParams* kp = (KParams*)uniform_u64((uint64_t)kp_in);                                             \
    const CAS int32_t* d = (const CAS int32_t*)uniform_u64((uint64_t)d_in);                           \
    LAS char* lds = (LAS char*)(uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_in); \
    const int32_t tw = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));                   \
    const int32_t lane = (int32_t)(threadIdx.x & 63);                                                 \
    Ctx c{kp, Smem(lds), d, __builtin_amdgcn_readfirstlane(task_in), tw, lane, tw - 1,                \
          kWaves - 1, tw * 64 + lane, kThreads, tw == 0};                                             \
    BODY                                                                                              \
  }

MKD_EXEC(exec_embed, return op_embed(c);)
MKD_EXEC(exec_qkv, return op_qkv<G::kHidden>(c);)
MKD_EXEC(exec_router, return op_rows_on_x<G::kHidden>(c, false);)
MKD_EXEC(exec_lm_head, return op_rows_on_x<G::kHidden>(c, true);)
MKD_EXEC(exec_moe_up, return op_moe_up<G::kHidden>(c);)
MKD_EXEC(exec_out, return (op_out<G::kHidden, G::kInter>(c));)
MKD_EXEC(exec_moe_down, return op_moe_down<G::kInter>(c);)
MKD_EXEC(exec_attn, return op_attn<G::kHd>(c);)

template <class G>
__device__ __forceinline__ bool run_task(KParams* kp, LAS char* lds, const CAS int32_t* d, int32_t task) {
  switch (d[D_OPCODE]) {
    case OP_EMBED: return exec_embed<G>(kp, lds, d, task);
    case OP_QKV: return exec_qkv<G>(kp, lds, d, task);
    case OP_ROUTER: return exec_router<G>(kp, lds, d, task);
    case OP_LM_HEAD: return exec_lm_head<G>(kp, lds, d, task);
    case OP_MOE_UP: return exec_moe_up<G>(kp, lds, d, task);
    case OP_OUT: return exec_out<G>(kp, lds, d, task);
    case OP_MOE_DOWN: return exec_moe_down<G>(kp, lds, d, task);
    case OP_ATTN: return exec_attn<G>(kp, lds, d, task);
    default: return true;
  }
}

// Trace record of a finished task (the controller's lane 0; fields in LDS were set by the
// task).  `list` = the workgroup.
__device__ __forceinline__ void trace_task(KParams* kp, LAS int32_t* mi, const CAS int32_t* d, uint64_t t0,
                                           bool leader, int list) {
  GAS uint64_t* trace = gas(kp->trace);
  if (trace && leader) {
    const int32_t gi = d[D_GIDX];
    if (gi >= 0 && gi < kp->trace_cap) {
      const uint64_t ready = ((uint64_t)(uint32_t)mi[MI_READY_HI] << 32) | (uint32_t)mi[MI_READY_LO];
      GAS uint64_t* r = trace + (int64_t)gi * 4;
      const uint64_t tend = wall_clock64();
      r[0] = t0;
      r[1] = ready ? ready : t0;
      r[2] = tend;
      // meta: opcode (8 bits) | list (12) | items (12) | staged - start (16, 10 ns) | done - start (16)
      const uint32_t st = mi[MI_T_STAGED] ? (uint32_t)mi[MI_T_STAGED] - (uint32_t)t0 : 0u;
      const uint32_t dn = mi[MI_T_DONE] ? (uint32_t)mi[MI_T_DONE] - (uint32_t)t0 : 0u;
      r[3] = (uint64_t)((uint32_t)d[D_OPCODE] & 0xFFu) | ((uint64_t)((uint32_t)list & 0xFFFu) << 8) |
             ((uint64_t)((uint32_t)mi[MI_ITEMS] & 0xFFFu) << 20) | ((uint64_t)min(st, 0xFFFFu) << 32) |
             ((uint64_t)min(dn, 0xFFFFu) << 48);
    }
  }
}

// Workgroup state that lives across tasks, set before the workgroup's first barrier: the
// workers read the routing-table layer and the claim entries, so their initial values
// must be visible before any task starts (LDS keeps the previous workgroup's contents).
__device__ __forceinline__ void init_team_state(LAS int32_t* mi, bool leader) {
  if (leader) {
    mi[MI_XS_LAYER] = -1;
    mi[MI_ROUTE_LAYER] = -1;
    mi[MI_WFAIL] = 0;
    for (int k = 0; k < 4; ++k) mi[MI_NEXT + k] = -1;
  }
}

// Controller-owned per-task state (no other wave reads it, so no barrier is needed).
__device__ __forceinline__ void reset_task_state(LAS int32_t* mi, bool leader) {
  if (leader) {
    mi[MI_ITEMS] = 0;
    mi[MI_READY_LO] = 0;
    mi[MI_READY_HI] = 0;
    mi[MI_T_STAGED] = 0;
    mi[MI_T_DONE] = 0;
  }
}

// Persistent interpreter: workgroup i walks task list i.  Every wave calls every task of
// the list; the tasks' own barriers keep the controller and the workers in step.
template <class G>
__global__ void __launch_bounds__(kThreads, 1) mk_persistent(Params prm) {
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  LAS char* lds = (LAS char*)lds_raw;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  const bool leader = threadIdx.x == 0;
  LAS int32_t* mi = Smem(lds).mi;
  init_team_state(mi, leader);
  __syncthreads();
  const int list = (int)blockIdx.x;
  const CAS int32_t* offs = cas(prm.cu_offsets);
  const int begin = offs[list], end = offs[list + 1];
  for (int t = begin; t < end; ++t) {
    // Opaque per task: argument fields are re-read (scalar cache) inside each task instead
    // of being hoisted out of the loop and kept live across every opcode body.
    uint64_t kpv = (uint64_t)kp;
    asm volatile("" : "+s"(kpv));
    KParams* kpt = (KParams*)kpv;
    const CAS int32_t* d = cas(kpt->tasks) + (int64_t)t * D_WORDS;
    // The next task's descriptor is touched now with a vector load, so that its scalar
    // loads at the next task's start find it in L2: a scalar miss that goes to HBM queues
    // behind the weight streams for microseconds.  The value is only consumed (waited
    // for) after this task.
#ifndef MKD_NO_DESC_PREFETCH
    int32_t dpre = 0;
    if (t + 1 < end && (threadIdx.x & 63) < 2)
      dpre = gas(kpt->tasks)[(int64_t)(t + 1) * D_WORDS + 16 * (threadIdx.x & 1)];
#endif
    reset_task_state(mi, leader);
    const uint64_t t0 = kpt->trace ? wall_clock64() : 0;
    const bool ok = run_task<G>(kpt, lds, d, t);
    trace_task(kpt, mi, d, t0, leader, list);
#ifndef MKD_NO_DESC_PREFETCH
    asm volatile("" ::"v"(dpre));
#endif
    if (!ok) break;
  }
}

// Ablation: one launch per wave of tasks; block i runs task first + i.
template <class G>
__global__ void __launch_bounds__(kThreads, 1) mk_wave(Params prm, int32_t first) {
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  LAS char* lds = (LAS char*)lds_raw;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  LAS int32_t* mi = Smem(lds).mi;
  init_team_state(mi, threadIdx.x == 0);
  reset_task_state(mi, threadIdx.x == 0);
  __syncthreads();
  const int32_t t = first + (int32_t)blockIdx.x;
  const CAS int32_t* d = cas(prm.tasks) + (int64_t)t * D_WORDS;
  const uint64_t t0 = prm.trace ? wall_clock64() : 0;
  run_task<G>(kp, lds, d, t);
  trace_task(kp, mi, d, t0, threadIdx.x == 0, (int)blockIdx.x);
}

__global__ void mk_clear(uint32_t* words, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    words[i] = 0u;
}

}  // namespace mkd

// ------------------------------------------------------------------ launch wrappers
namespace mkd {

hipError_t launch_clear(uint32_t* words, int64_t n, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>(1024, std::max<int64_t>(1, (n + 255) / 256));
  hipLaunchKernelGGL(mk_clear, dim3((unsigned)blocks), dim3(256), 0, s, words, n);
  return hipGetLastError();
}

// Geometry instance of a configuration: 0 = full (hidden 2048), 1 = tiny (hidden 256), -1 = none.
int geometry_index(int hidden, int inter, int hd) {
  if (hidden == GeomFull::kHidden && inter == GeomFull::kInter && hd == GeomFull::kHd) return 0;
  if (hidden == GeomTiny::kHidden && inter == GeomTiny::kInter && hd == GeomTiny::kHd) return 1;
  return -1;
}

hipError_t launch_persistent(const Params& p, int n_wg, hipStream_t s) {
  void* args[] = {const_cast<Params*>(&p)};
  const int gi = geometry_index(p.hidden, p.inter, p.head_dim);
  if (gi < 0) return hipErrorInvalidValue;
  const void* fn = gi == 0 ? reinterpret_cast<const void*>(&mk_persistent<GeomFull>)
                           : reinterpret_cast<const void*>(&mk_persistent<GeomTiny>);
  return hipLaunchCooperativeKernel(fn, dim3(n_wg), dim3(kThreads),
                                    args, 0, s);
}

hipError_t launch_wave(const Params& p, int32_t first, int32_t count, hipStream_t s) {
  const int gi = geometry_index(p.hidden, p.inter, p.head_dim);
  if (gi == 0) hipLaunchKernelGGL(mk_wave<GeomFull>, dim3(count), dim3(kThreads), 0, s, p, first);
  else if (gi == 1) hipLaunchKernelGGL(mk_wave<GeomTiny>, dim3(count), dim3(kThreads), 0, s, p, first);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

int threads_per_wg() { return kThreads; }

}  // namespace mkd
