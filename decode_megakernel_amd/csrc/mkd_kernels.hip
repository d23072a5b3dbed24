// mkd_kernels.hip - the decode megakernel for gfx950: tile bodies of every opcode and
// the persistent task interpreter (plus the op-per-kernel ablation launcher).
//
// Method: "Inside the megakernel serving engine for North Mini Code" (Cohere).
//  - "What is a Megakernel?": one workgroup per compute unit, resident for the whole
//    step, walking a host-built task list in global memory; dependencies are counters
//    that producers increment and consumers spin on.
//  - "Tasks": the GEMM opcodes share one body (here: a bf16 GEMV tile streaming its
//    weight rows into registers with 16-byte non-temporal loads, fp32 accumulation,
//    wave reductions); QKV applies RoPE in the epilogue; attention is split over KV
//    slices and combined; routing scores the experts and picks the top-k per token;
//    expert gate/up fuses SiLU-and-multiply; MOE_COMBINE weights expert outputs by
//    router scores.
//  - "Weight prefetch" (section "Where the speedup comes from", item 3): weights
//    never depend on this step's activations, so every tile issues its weight loads
//    before it waits on its input counter.
//  - "The task scheduler": the attention and MoE stages are drained by claimer tasks
//    that atomically take the next item of a shared queue until it is empty.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mkd_common.h"
#include "mkd_device.h"

namespace mkd {

// ------------------------------------------------------------------ LDS layout
// One workgroup per CU is forced by the LDS footprint (> half of the 160 KB).
constexpr int kLdsXs = 0;            // 128 KB: activation staging, attention merge, logits
constexpr int kLdsXsBytes = 131072;
constexpr int kLdsRowsum = 131072;   // 8 KB: per-row results of a tile
constexpr int kLdsRoute = 139264;    // 8 KB: routing tables
constexpr int kLdsMisc = 147456;     // 1 KB: broadcasts, inverse RMS
constexpr int kLdsBytes = 148480;
constexpr int kMaxKv = 16;            // KV groups handled by the residual finalisation
constexpr int kMaxDs = 16;            // MoE-down splits handled by the residual finalisation
constexpr int kAttnMaxChunks = 1536;  // attention chunks per (sequence, KV group) combined in LDS

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
        mf(reinterpret_cast<LAS float*>(base + kLdsMisc + 512)) {}
};
// misc int slots
constexpr int MI_BCAST = 0;
constexpr int MI_OK = 1;
constexpr int MI_WAIT_CTR = 2;   // last satisfied wait of this workgroup (skip repeats)
constexpr int MI_WAIT_TGT = 3;
constexpr int MI_ITEMS = 4;      // trace: items claimed by the current task
constexpr int MI_READY_LO = 6;   // trace: when the current task's first wait completed
constexpr int MI_READY_HI = 7;
constexpr int MI_TOK = 16;  // [16] token list of the current GEMV

// Routing table offsets inside Smem::route (int32 units; at most B*k <= 256 entries
// and min(E, B*k) <= 256 active experts).
constexpr int RT_IDS = 0;       // [16][16] selected experts per token
constexpr int RT_W = 256;       // [16][16] routing weights (float bits)
constexpr int RT_NACT = 512;    // number of active experts
constexpr int RT_ACT = 520;     // [256] active experts, ascending
constexpr int RT_OFF = 776;     // [257] CSR offsets of each active expert's (token, slot) list
constexpr int RT_FLAT = 1036;   // [256] b*k + j entries, experts ascending, tokens ascending
constexpr int RT_SCAN = 1292;   // [16] block-scan scratch

// ------------------------------------------------------------------ task context
struct Ctx {
  KParams* kp;           // kernel arguments (constant segment)
  Smem s;
  const GAS int32_t* d;  // descriptor
  int32_t task;          // global task index
};

__device__ __forceinline__ GAS uint32_t* layer_ctr(const DParams& p, int l, int off) {
  return p.counters + (int64_t)l * p.ctr.per_layer + off;
}

// Spin until counter >= target (thread 0 polls, then acquire; whole workgroup
// returns together).  A wait this workgroup already saw satisfied is skipped
// (counters only grow during a step).  Returns false when the step is aborted.
__device__ __forceinline__ bool mk_wait(Ctx& c, GAS uint32_t* ctr, uint32_t target) {
  const DParams p = device_view(*c.kp);
  const int32_t idx = (int32_t)(ctr - p.counters);
  if (threadIdx.x == 0) {
    int ok = 1;
    if (!(c.s.mi[MI_WAIT_CTR] == idx && target <= (uint32_t)c.s.mi[MI_WAIT_TGT])) {
      int32_t spins = 0;
      uint32_t v;
      while ((v = ctr_load(ctr)) < target) {
        if ((spins & 63) == 63 && aborted(p)) { ok = 0; break; }
        if (++spins > c.kp->spin_limit) {
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
    c.s.mi[MI_OK] = ok;
  }
  __syncthreads();
  return c.s.mi[MI_OK] != 0;
}

// Publish this workgroup's stores and add one to the counter; returns the old value.
__device__ __forceinline__ uint32_t mk_arrive(Ctx& c, GAS uint32_t* ctr) {
  wait_vm_all();
  __syncthreads();
  if (threadIdx.x == 0) {
    fence_release_agent();
    c.s.mi[MI_BCAST] = (int32_t)ctr_add(ctr, 1u);
  }
  __syncthreads();
  return (uint32_t)c.s.mi[MI_BCAST];
}

// Claim the next item of a shared queue (one atomic per claim, broadcast).
__device__ __forceinline__ int32_t mk_claim(Ctx& c, GAS uint32_t* head) {
  __syncthreads();
  if (threadIdx.x == 0) {
    c.s.mi[MI_BCAST] = (int32_t)ctr_add(head, 1u);
    c.s.mi[MI_ITEMS] += 1;
  }
  __syncthreads();
  return c.s.mi[MI_BCAST];
}

// ------------------------------------------------------------------ GEMV tile
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

// Lane mapping of a K-long bf16 row onto a wave: LPR lanes per row, CPL 16-byte
// chunks per lane per row, RPS rows per wave step; wave w takes steps w, w+8, ...
template <int K>
struct Gemv {
  static constexpr int CH = K / 8;
  static constexpr int LPR = (CH % 64 == 0) ? 64 : (CH % 32 == 0) ? 32 : (CH % 16 == 0) ? 16 : 8;
  static constexpr int RPS = 64 / LPR;
  static constexpr int CPL = CH / LPR;
  static constexpr int MAXS = kWreg / CPL;
  static constexpr int MAX_ROWS = MAXS * RPS * kWaves;
  static_assert(K % 64 == 0, "row length must be a multiple of 64");
};

template <int K>
__device__ __forceinline__ void gemv_load(u32x4 (&wb)[kWreg], const RowSrc& src, int R) {
  using G = Gemv<K>;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int si = 0; si < G::MAXS; ++si) {
    const int row = (w + kWaves * si) * G::RPS + lane / G::LPR;
#pragma unroll
    for (int c = 0; c < G::CPL; ++c) {
      const int kc = lane % G::LPR + G::LPR * c;
      if (row < R) wb[si * G::CPL + c] = ld_stream16(src.row(row) + kc * 8);
      else wb[si * G::CPL + c] = u32x4{0, 0, 0, 0};
    }
  }
}

// rowsum[row * nb + j] = W[row] . x_j for rows < R and activation vectors j < nb,
// where x_j = xs + tok[j] * K (tok in LDS).
template <int K>
__device__ __forceinline__ void gemv_compute(const u32x4 (&wb)[kWreg], const LAS float* xs,
                                             const LAS int32_t* tok, int nb, int R, LAS float* rowsum) {
  using G = Gemv<K>;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int si = 0; si < G::MAXS; ++si) {
    const int row = (w + kWaves * si) * G::RPS + lane / G::LPR;
    if ((w + kWaves * si) * G::RPS >= R) break;  // wave-uniform
    for (int j = 0; j < nb; ++j) {
      const LAS float* x = xs + tok[j] * K;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < G::CPL; ++c) {
        const int kc = lane % G::LPR + G::LPR * c;
        const LAS f32x4* xp = reinterpret_cast<const LAS f32x4*>(x + kc * 8);
        acc += dot8(wb[si * G::CPL + c], xp[0], xp[1]);
      }
      acc = group_sum<G::LPR>(acc);
      if (lane % G::LPR == 0 && row < R) rowsum[row * nb + j] = acc;
    }
  }
}

// ------------------------------------------------------------------ activation staging
// inverse RMS of the residual rows h_l[b] from the per-row-tile sums of squares.
__device__ __forceinline__ void stage_inv_rms(Ctx& c, int l) {
  const DParams p = device_view(*c.kp);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = w; b < p.batch; b += kWaves) {
    const GAS float* ss = p.ss + ((int64_t)l * p.max_batch + b) * p.shape.n_rt;
    float t = 0.0f;
    for (int r = lane; r < p.shape.n_rt; r += 64) t += ss[r];
    t = group_sum<64>(t);
    if (lane == 0) c.s.mf[b] = 1.0f / sqrtf(t / (float)p.hidden + p.rms_eps);
  }
  __syncthreads();
}

// xs[b][k] = h_l[b][k] * inv_rms[b] * gamma_l[k] for every token of the batch
// (the RMSNorm every consumer of layer l's input applies on the fly).
__device__ __forceinline__ void stage_x_normed(Ctx& c, int l) {
  const DParams p = device_view(*c.kp);
  stage_inv_rms(c, l);
  const int H = p.hidden;
  const GAS uint16_t* gamma = p.norm + (int64_t)l * H;
  const int n8 = p.batch * (H / 8);
  for (int i = threadIdx.x; i < n8; i += kThreads) {
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
    LAS float* xo = c.s.xs + (int64_t)b * H + k8;
    *reinterpret_cast<LAS f32x4*>(xo) = o0;
    *reinterpret_cast<LAS f32x4*>(xo + 4) = o1;
  }
  if (threadIdx.x < 16) c.s.mi[MI_TOK + threadIdx.x] = threadIdx.x;
  __syncthreads();
}

// ------------------------------------------------------------------ residual finalisation
// The fused residual add + RMSNorm at the end of a layer ("Where the speedup comes
// from": parallel layers are rejoined only by it).  The last arriver of residual
// row tile rt writes h_{l+1} = h_l + sum_g a_g + sum_ds m_ds for those rows and
// their sum of squares; consumers of layer l+1 normalise on the fly.
__device__ __forceinline__ bool finalize_rows(Ctx& c, int l, int rt) {
  const DParams p = device_view(*c.kp);
  fence_acquire_agent();
  const int R = p.shape.rt_rows, H = p.hidden, B = p.batch;
  const int r0 = rt * R;
  LAS float* red = c.s.rowsum;  // [B][R] squares
  const int64_t hstride = (int64_t)p.max_batch * H;
  for (int i = threadIdx.x; i < B * R; i += kThreads) {
    const int b = i / R, r = r0 + i % R;
    const int64_t hb = (int64_t)b * H + r;
    // independent loads in batches (h, O-proj splits, MoE-down splits), summed in order
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
    p.h[(int64_t)(l + 1) * hstride + hb] = v;
    red[i] = v * v;
  }
  __syncthreads();
  if (threadIdx.x < B) {
    float t = 0.0f;
    for (int r = 0; r < R; ++r) t += red[threadIdx.x * R + r];
    p.ss[((int64_t)(l + 1) * p.max_batch + threadIdx.x) * p.shape.n_rt + rt] = t;
  }
  mk_arrive(c, layer_ctr(p, l + 1, p.ctr.x_ready));
  return true;
}

// Arrive on a residual row tile; the last of its n_kv + n_ds producers finalises it.
__device__ __forceinline__ bool arrive_rt(Ctx& c, int l, int rt) {
  const DParams p = device_view(*c.kp);
  const uint32_t old = mk_arrive(c, layer_ctr(p, l, p.ctr.rt + rt));
  if (old + 1 == (uint32_t)(p.n_kv + p.shape.n_ds)) return finalize_rows(c, l, rt);
  return true;
}

// ------------------------------------------------------------------ OP_EMBED
__device__ __forceinline__ bool op_embed(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int rt = c.d[D_ARG0];
  const int R = p.shape.rt_rows, H = p.hidden, B = p.batch;
  LAS float* red = c.s.rowsum;
  for (int i = threadIdx.x; i < B * R; i += kThreads) {
    const int b = i / R, r = rt * R + i % R;
    int tok = p.tokens[b];
    if (tok < 0 || tok >= p.vocab) {
      report_error(p, 2u, c.task, -1, (uint32_t)tok, (uint32_t)p.vocab);
      tok = 0;
    }
    const float v = bf16_to_f32(p.embed[(int64_t)tok * H + r]);
    p.h[(int64_t)b * H + r] = v;
    red[i] = v * v;
  }
  __syncthreads();
  if (threadIdx.x < B) {
    float t = 0.0f;
    for (int r = 0; r < R; ++r) t += red[threadIdx.x * R + r];
    p.ss[(int64_t)threadIdx.x * p.shape.n_rt + rt] = t;
  }
  mk_arrive(c, layer_ctr(p, 0, p.ctr.x_ready));
  return true;
}

// ------------------------------------------------------------------ OP_QKV
// Tile = head hh of the q|k|v rows, dims [j0, j0+PB) and [j0+hd/2, j0+hd/2+PB), so
// every RoPE pair (i, i+hd/2) is in the tile.  Epilogue: RoPE at the token's
// position (angles in fp64), q to the workspace, k and v as bf16 into the paged-KV
// slot (page_table[b][pos/page], pos%page) of this layer.
template <int K>
__device__ __forceinline__ bool op_qkv(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], hh = c.d[D_ARG0], j0 = c.d[D_ARG1], PB = c.d[D_ARG2];
  const int hd = p.head_dim, half = hd / 2, H = p.hidden;
  const GAS uint16_t* wl = p.w_qkv + (int64_t)l * (p.n_q + 2 * p.n_kv) * hd * H;
  const RowSrc src{wl + ((int64_t)hh * hd + j0) * H, wl + ((int64_t)hh * hd + half + j0) * H, H, PB};
  u32x4 wb[kWreg];
  gemv_load<K>(wb, src, 2 * PB);
  if (!mk_wait(c, device_view(*c.kp).counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  stage_x_normed(c, l);
  const int B = p.batch;
  gemv_compute<K>(wb, c.s.xs, c.s.mi + MI_TOK, B, 2 * PB, c.s.rowsum);
  __syncthreads();
  for (int i = threadIdx.x; i < PB * B; i += kThreads) {
    const int r = i / B, b = i % B, dim = j0 + r;
    const float a = c.s.rowsum[r * B + b], bb = c.s.rowsum[(PB + r) * B + b];
    const int pos = p.seq_lens[b];
    float o1 = a, o2 = bb;
    if (hh < p.n_q + p.n_kv) {
      const double ang = (double)pos * p.inv_freq[dim];
      const float cs = (float)cos(ang), sn = (float)sin(ang);
      o1 = a * cs - bb * sn;
      o2 = bb * cs + a * sn;
    }
    if (hh < p.n_q) {
      GAS float* q = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * hd + (int64_t)hh * hd;
      q[dim] = o1;
      q[dim + half] = o2;
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
        base[(int64_t)t * hd + dim] = f32_to_bf16(o1);
        base[(int64_t)t * hd + dim + half] = f32_to_bf16(o2);
      } else {
        base[(int64_t)dim * p.page + t] = f32_to_bf16(o1);
        base[(int64_t)(dim + half) * p.page + t] = f32_to_bf16(o2);
      }
    }
  }
  mk_arrive(c, device_view(*c.kp).counters + c.d[D_SIGNAL]);
  return true;
}

// ------------------------------------------------------------------ OP_ROUTER / OP_LM_HEAD
// Plain GEMV tiles on the normed input: router logits (layer l) or vocabulary logits
// (final norm, tied embedding).
template <int K>
__device__ __forceinline__ bool op_rows_on_x(Ctx& c, bool lm_head) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], r0 = c.d[D_ARG0], R = c.d[D_ARG1];
  const int H = p.hidden;
  const GAS uint16_t* base = lm_head ? p.embed + (int64_t)r0 * H
                                 : p.w_router + ((int64_t)l * p.n_experts + r0) * H;
  const RowSrc src{base, base, H, R};
  u32x4 wb[kWreg];
  gemv_load<K>(wb, src, R);
  if (!mk_wait(c, device_view(*c.kp).counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  stage_x_normed(c, l);
  const int B = p.batch;
  gemv_compute<K>(wb, c.s.xs, c.s.mi + MI_TOK, B, R, c.s.rowsum);
  __syncthreads();
  for (int i = threadIdx.x; i < R * B; i += kThreads) {
    const int r = i / B, b = i % B;
    if (lm_head) p.logits[(int64_t)b * p.vocab + r0 + r] = c.s.rowsum[i];
    else p.router[((int64_t)l * p.max_batch + b) * p.n_experts + r0 + r] = c.s.rowsum[i];
  }
  if (c.d[D_SIGNAL] >= 0) mk_arrive(c, device_view(*c.kp).counters + c.d[D_SIGNAL]);
  return true;
}

// ------------------------------------------------------------------ OP_OPROJ
// Split-K over KV groups (Figure 7: O-proj for a KV group starts as soon as that
// group's attention output lands): rows [rt*R, +R) of W_o, columns of group g.
template <int K>
__device__ __forceinline__ bool op_oproj(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER], rt = c.d[D_ARG0], g = c.d[D_ARG1];
  const int R = p.shape.rt_rows, H = p.hidden, KO = p.n_q * p.head_dim;
  const GAS uint16_t* base = p.w_o + ((int64_t)l * H + (int64_t)rt * R) * KO + (int64_t)g * K;
  const RowSrc src{base, base, KO, R};
  u32x4 wb[kWreg];
  gemv_load<K>(wb, src, R);
  if (!mk_wait(c, device_view(*c.kp).counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  const int B = p.batch;
  for (int i = threadIdx.x; i < B * (K / 4); i += kThreads) {
    const int b = i / (K / 4), k4 = (i % (K / 4)) * 4;
    *reinterpret_cast<LAS f32x4*>(c.s.xs + b * K + k4) =
        *reinterpret_cast<const GAS f32x4*>(p.attn_o + ((int64_t)l * p.max_batch + b) * KO +
                                         (int64_t)g * K + k4);
  }
  if (threadIdx.x < 16) c.s.mi[MI_TOK + threadIdx.x] = threadIdx.x;
  __syncthreads();
  gemv_compute<K>(wb, c.s.xs, c.s.mi + MI_TOK, B, R, c.s.rowsum);
  __syncthreads();
  for (int i = threadIdx.x; i < R * B; i += kThreads) {
    const int r = i / B, b = i % B;
    p.a_part[(((int64_t)l * p.n_kv + g) * p.max_batch + b) * H + rt * R + r] = c.s.rowsum[i];
  }
  return arrive_rt(c, l, rt);
}

// ------------------------------------------------------------------ routing
// Exclusive prefix sum of one int per thread over the workgroup; *total receives the
// sum.  tmp: kWaves ints of LDS.
__device__ __forceinline__ int block_exscan(int v, LAS int32_t* tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = tmp[i];
    pre += i < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// ROUTER_TOPK + ROUTE_FINALIZE + MOE_GATHER in LDS: top-k of each token's router
// logits (descending, ties to the lower expert index), softmax over the selected
// logits, then the active experts in ascending order and, per expert, its
// (token, slot) entries in ascending token order.
__device__ __forceinline__ bool route_layer(Ctx& c, int l, bool write_debug) {
  const DParams p = device_view(*c.kp);
  const int B = p.batch, E = p.n_experts, k = p.top_k;
  LAS int32_t* rt = c.s.route;
  LAS float* rw = reinterpret_cast<LAS float*>(rt + RT_W);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = w; b < B; b += kWaves) {
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
        const float e = expf(rw[b * 16 + j] - sel_v0);
        rw[b * 16 + j] = e;
        sum += e;
      }
      for (int j = 0; j < k; ++j) rw[b * 16 + j] /= sum;
    }
  }
  __syncthreads();
  // per-expert entry counts, one thread per expert, then block-wide exclusive scans
  // give each active expert its rank and its offset in the flat (token, slot) list.
  const int e = threadIdx.x;
  int m_e = 0;
  if (e < E)
    for (int b = 0; b < B; ++b)
      for (int j = 0; j < k; ++j) m_e += rt[RT_IDS + b * 16 + j] == e;
  int n_entries = 0, n_act = 0;
  const int off = block_exscan(m_e, rt + RT_SCAN, n_entries);
  const int rank = block_exscan(m_e > 0 ? 1 : 0, rt + RT_SCAN, n_act);
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
  __syncthreads();
  return true;
}

// ------------------------------------------------------------------ OP_MOE_UP (claimer)
// Claims (active expert, tile of up_rows activation rows); weights = up_rows gate
// rows and the matching up rows; epilogue silu(gate) * up for every token routed to
// the expert; arrives on the expert's up counter.
template <int K>
__device__ __forceinline__ bool op_moe_up(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  if (!mk_wait(c, device_view(*c.kp).counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  route_layer(c, l, c.d[D_ARG0] == 0);
  stage_x_normed(c, l);
  const LAS int32_t* rt = c.s.route;
  const int n_act = rt[RT_NACT];
  const int UR = p.shape.up_rows, NT = p.shape.n_up_tiles, H = p.hidden, I = p.inter;
  const int k = p.top_k;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.up_claim);
  for (;;) {
    const int idx = mk_claim(c, head);
    if (idx >= n_act * NT) break;
    const int a = idx / NT, tile = idx % NT;
    const int e = rt[RT_ACT + a];
    const GAS uint16_t* base = p.w_gate_up + (((int64_t)l * p.n_experts + e) * 2 * I + (int64_t)tile * UR) * H;
    const RowSrc src{base, base + (int64_t)I * H, H, UR};
    u32x4 wb[kWreg];
    gemv_load<K>(wb, src, 2 * UR);
    const int o0 = rt[RT_OFF + a], n_e = rt[RT_OFF + a + 1] - o0;
    if (threadIdx.x < n_e) c.s.mi[MI_TOK + threadIdx.x] = rt[RT_FLAT + o0 + threadIdx.x] / k;
    __syncthreads();
    gemv_compute<K>(wb, c.s.xs, c.s.mi + MI_TOK, n_e, 2 * UR, c.s.rowsum);
    __syncthreads();
    for (int i = threadIdx.x; i < UR * n_e; i += kThreads) {
      const int r = i / n_e, j = i % n_e;
      const float g = c.s.rowsum[r * n_e + j], u = c.s.rowsum[(UR + r) * n_e + j];
      const float act = g / (1.0f + expf(-g)) * u;
      const int slot = rt[RT_FLAT + o0 + j];  // b * k + j
      p.moe_act[((int64_t)l * p.max_batch * k + slot) * I + (int64_t)tile * UR + r] = act;
    }
    mk_arrive(c, layer_ctr(p, l, p.ctr.up_done + e));
  }
  return true;
}

// ------------------------------------------------------------------ OP_MOE_DOWN (claimer)
// Claims (residual row tile rt, expert split ds): for each active expert of the split
// (every n_ds-th in ascending order) it streams W_down[e][rows of rt] (issued before
// waiting for that expert's up tiles), computes y_e for the expert's tokens and
// accumulates w_{b,e} * y_e into the split's partial m_ds[b][rows]; the last producer
// of the row tile finalises the residual.
template <int K>
__device__ __forceinline__ bool op_moe_down(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  if (!mk_wait(c, device_view(*c.kp).counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  route_layer(c, l, false);
  const LAS int32_t* rt = c.s.route;
  const LAS float* rw = reinterpret_cast<const LAS float*>(rt + RT_W);
  const int n_act = rt[RT_NACT];
  const int R = p.shape.rt_rows, NDS = p.shape.n_ds, H = p.hidden, I = p.inter, B = p.batch;
  const int k = p.top_k;
  LAS float* macc = c.s.rowsum + 1024;  // [R][B]
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.down_claim);
  for (;;) {
    const int idx = mk_claim(c, head);
    if (idx >= p.shape.n_rt * NDS) break;
    const int rtile = idx / NDS, ds = idx % NDS;
    for (int i = threadIdx.x; i < R * B; i += kThreads) macc[i] = 0.0f;
    for (int a = ds; a < n_act; a += NDS) {
      const int e = rt[RT_ACT + a];
      const GAS uint16_t* base = p.w_down + (((int64_t)l * p.n_experts + e) * H + (int64_t)rtile * R) * I;
      const RowSrc src{base, base, I, R};
      u32x4 wb[kWreg];
      gemv_load<K>(wb, src, R);
      if (!mk_wait(c, layer_ctr(p, l, p.ctr.up_done + e), (uint32_t)p.shape.n_up_tiles)) return false;
      const int o0 = rt[RT_OFF + a], n_e = rt[RT_OFF + a + 1] - o0;
      for (int i = threadIdx.x; i < n_e * (K / 4); i += kThreads) {
        const int j = i / (K / 4), k4 = (i % (K / 4)) * 4;
        const int slot = rt[RT_FLAT + o0 + j];
        *reinterpret_cast<LAS f32x4*>(c.s.xs + j * K + k4) =
            *reinterpret_cast<const GAS f32x4*>(p.moe_act + ((int64_t)l * p.max_batch * k + slot) * I + k4);
      }
      if (threadIdx.x < n_e) c.s.mi[MI_TOK + threadIdx.x] = threadIdx.x;
      __syncthreads();
      gemv_compute<K>(wb, c.s.xs, c.s.mi + MI_TOK, n_e, R, c.s.rowsum);
      __syncthreads();
      for (int i = threadIdx.x; i < R * n_e; i += kThreads) {
        const int r = i / n_e, j = i % n_e;
        const int slot = rt[RT_FLAT + o0 + j];
        const int b = slot / k, sj = slot % k;
        macc[r * B + b] += rw[b * 16 + sj] * c.s.rowsum[r * n_e + j];
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < R * B; i += kThreads) {
      const int r = i / B, b = i % B;
      p.m_part[(((int64_t)l * NDS + ds) * p.max_batch + b) * H + (int64_t)rtile * R + r] = macc[i];
    }
    if (!arrive_rt(c, l, rtile)) return false;
  }
  return true;
}

// ------------------------------------------------------------------ OP_ATTN (claimer)
// Paged GQA decode attention, split over pages ("Tasks": ATTN_DECODE over a partial
// KV slice, ATTN_COMBINE merging the partials; ATTN_DRAIN claiming from the queue).
// One item = (sequence b, KV group g, chunk of pages_per_item pages); each wave of
// the workgroup takes every 8th page of the chunk.  Per 16-token page:
//   S^T[t][h] = K[t][:] . Qs^T[:][h]   (v_mfma_f32_16x16x32_bf16, tokens x heads,
//                                        Qs = q * log2(e)/sqrt(hd) in bf16)
//   online softmax in base 2 per head, P in bf16
//   O^T[d][h] += V^T[d][t] P^T[t][h]    (v_mfma_f32_16x16x16_bf16; V pages are stored
//                                        dim-major so V^T rows are contiguous)
// The cached pages are streamed before waiting for this layer's QKV tiles; only the
// page holding the new token is read after the wait.
template <int HD, int MAXP>
__device__ __forceinline__ bool attn_item(Ctx& c, int l, int idx, bool& waited) {
  const DParams p = device_view(*c.kp);
  const int B = p.batch, nkv = p.n_kv, ppi = p.shape.pages_per_item;
  // map idx -> (b, g, chunk)
  int b = -1, g = 0, chunk = 0, nchunks = 0, base_bg = 0;
  {
    int acc = 0;
    for (int bb = 0; bb < B; ++bb) {
      const int npg = p.seq_lens[bb] / p.page + 1;
      const int nit = (npg + ppi - 1) / ppi;
      if (idx < acc + nit * nkv) {
        const int local = idx - acc;
        b = bb;
        g = local / nit;
        chunk = local % nit;
        nchunks = nit;
        base_bg = acc + g * nit;
        break;
      }
      acc += nit * nkv;
    }
  }
  if (b < 0) return true;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pos = p.seq_lens[b];
  const int npg = pos / p.page + 1, last = npg - 1;
  const int c0 = chunk * ppi, c1 = min(npg, c0 + ppi);
  constexpr int NK = HD / 32, NV = HD / 16;
  u32x4 kr[MAXP][NK];
  u32x2 vr[MAXP][NV];
  int lp[MAXP];
  int64_t kbase[MAXP], vbase[MAXP];
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    lp[i] = c0 + w + kWaves * i;
    kbase[i] = -1;
    vbase[i] = -1;
    if (lp[i] < c1) {
      const int phys = lp[i] < p.max_pages ? p.page_table[(int64_t)b * p.max_pages + lp[i]] : -1;
      if (phys < 0 || phys >= p.n_pages) {
        if (lane == 0) report_error(p, 2u, c.task, -1, (uint32_t)phys, (uint32_t)p.n_pages);
        lp[i] = c1;  // skip
      } else {
        kbase[i] = ((((int64_t)l * 2 + 0) * p.n_pages + phys) * nkv + g) * (int64_t)p.page * HD;
        vbase[i] = ((((int64_t)l * 2 + 1) * p.n_pages + phys) * nkv + g) * (int64_t)p.page * HD;
      }
    }
    if (lp[i] < c1 && lp[i] != last) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        kr[i][kk] = ld_stream16(p.kv_pool + kbase[i] + (lane & 15) * HD + kk * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int dt = 0; dt < NV; ++dt)
        vr[i][dt] = ld_stream8(p.kv_pool + vbase[i] + (dt * 16 + (lane & 15)) * 16 + (lane >> 4) * 4);
    }
  }
  if (!waited) {
    if (!mk_wait(c, device_view(*c.kp).counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
    waited = true;
  }
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    if (lp[i] < c1 && lp[i] == last) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        kr[i][kk] = *reinterpret_cast<const GAS u32x4*>(p.kv_pool + kbase[i] + (lane & 15) * HD + kk * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int dt = 0; dt < NV; ++dt)
        vr[i][dt] = *reinterpret_cast<const GAS u32x2*>(p.kv_pool + vbase[i] + (dt * 16 + (lane & 15)) * 16 + (lane >> 4) * 4);
    }
  }
  // Q^T operand: lane holds head (lane & 15), dims kk*32 + (lane>>4)*8 + [0, 8)
  const int hpg = p.n_q / nkv;
  const int head = lane & 15;
  const float qscale = 1.4426950408889634f / sqrtf((float)HD);
  u32x4 qb[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (head < hpg) {
      const GAS float* qp = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * HD +
                        (int64_t)(g * hpg + head) * HD + kk * 32 + (lane >> 4) * 8;
      const f32x4 a0 = *reinterpret_cast<const GAS f32x4*>(qp);
      const f32x4 a1 = *reinterpret_cast<const GAS f32x4*>(qp + 4);
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
        if (lp[i] * p.page + (lane >> 4) * 4 + r > pos) s[r] = -INFINITY;
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
  // per-wave results -> LDS: mw[w][16], lw[w][16], ow[w][hpg][HD]
  LAS float* mw = c.s.xs;
  LAS float* lw = c.s.xs + kWaves * 16;
  LAS float* ow = c.s.xs + 2 * kWaves * 16;
  if (lane < 16) {
    mw[w * 16 + lane] = m;
    lw[w * 16 + lane] = lsum;
  }
  if (head < hpg) {
#pragma unroll
    for (int dt = 0; dt < NV; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ow[(w * hpg + head) * HD + dt * 16 + (lane >> 4) * 4 + r] = o[dt][r];
  }
  __syncthreads();
  // merge the waves: unnormalised o, running max m and sum l per head
  GAS float* part = p.attn_part + (int64_t)idx * hpg * (HD + 2);
  for (int t = threadIdx.x; t < hpg * HD; t += kThreads) {
    const int h = t / HD, dd = t % HD;
    float M = -INFINITY;
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mw[ww * 16 + h]);
    float acc = 0.0f, L = 0.0f;
    for (int ww = 0; ww < kWaves; ++ww) {
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
  const uint32_t old = mk_arrive(c, layer_ctr(p, l, p.ctr.attn_items + b * nkv + g));
  if (old + 1 == (uint32_t)nchunks) {
    // last item of (b, g): combine all chunks (log-sum-exp merge, chunk order fixed)
    fence_acquire_agent();
    const GAS float* pb = p.attn_part + (int64_t)base_bg * hpg * (HD + 2);
    LAS float* scl = c.s.xs;                       // [nchunks][hpg] merged weights
    LAS float* mrow = c.s.xs + kAttnMaxChunks * 16;  // [hpg] max, then [hpg] denominators
    for (int h = w; h < hpg; h += kWaves) {
      float M = -INFINITY;
      for (int ci = lane; ci < nchunks; ci += 64) M = fmaxf(M, pb[((int64_t)ci * hpg + h) * (HD + 2) + HD]);
      M = wave_max(M);
      float den = 0.0f;
      for (int ci = lane; ci < nchunks; ci += 64) {
        const GAS float* pc = pb + ((int64_t)ci * hpg + h) * (HD + 2);
        const float sc = exp2f(pc[HD] - M);
        scl[ci * hpg + h] = sc;
        den += sc * pc[HD + 1];
      }
      den = group_sum<64>(den);
      if (lane == 0) mrow[h] = 1.0f / den;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < hpg * (HD / 4); t += kThreads) {
      const int h = t / (HD / 4), d4 = (t % (HD / 4)) * 4;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nchunks; c0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (c0 + j < nchunks) v[j] = *reinterpret_cast<const GAS f32x4*>(pb + ((int64_t)(c0 + j) * hpg + h) * (HD + 2) + d4);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float sc = c0 + j < nchunks ? scl[(c0 + j) * hpg + h] : 0.0f;
          acc.x += sc * v[j].x;
          acc.y += sc * v[j].y;
          acc.z += sc * v[j].z;
          acc.w += sc * v[j].w;
        }
      }
      const float inv = mrow[h];
      GAS float* dst = p.attn_o + ((int64_t)l * p.max_batch + b) * p.n_q * HD + (int64_t)(g * hpg + h) * HD + d4;
      *reinterpret_cast<GAS f32x4*>(dst) = f32x4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    }
    mk_arrive(c, layer_ctr(p, l, p.ctr.comb + g));
  }
  return true;
}

template <int HD>
__device__ __forceinline__ bool op_attn(Ctx& c) {
  const DParams p = device_view(*c.kp);
  const int l = c.d[D_LAYER];
  int n_items = 0;
  for (int b = 0; b < p.batch; ++b)
    n_items += ((p.seq_lens[b] / p.page + 1 + p.shape.pages_per_item - 1) / p.shape.pages_per_item) * p.n_kv;
  if (n_items > p.max_attn_items) n_items = p.max_attn_items;
  GAS uint32_t* head = layer_ctr(p, l, p.ctr.attn_claim);
  bool waited = false;
  for (;;) {
    const int idx = mk_claim(c, head);
    if (idx >= n_items) break;
    if (!attn_item<HD, 2>(c, l, idx, waited)) return false;
    __syncthreads();
  }
  return true;
}

// ------------------------------------------------------------------ dispatch
// One non-inlined function per opcode: each gets its own register allocation, and
// nothing but the task index lives across tasks in the interpreter loop.
#define MKD_CASE_K(KV, CALL) \
  case KV: {                 \
    constexpr int K = KV;    \
    return CALL;             \
  }

#define MKD_EXEC(NAME, BODY)                                                                     \
  __device__ __noinline__ bool NAME(KParams* kp, LAS char* lds, const GAS int32_t* d, int32_t task) { \
    Ctx c{kp, Smem(lds), d, task};                                                               \
    BODY                                                                                         \
  }

MKD_EXEC(exec_embed, return op_embed(c);)
MKD_EXEC(exec_qkv, switch (kp->hidden) { MKD_CASE_K(256, op_qkv<K>(c)) MKD_CASE_K(2048, op_qkv<K>(c)) } return false;)
MKD_EXEC(exec_router, switch (kp->hidden) { MKD_CASE_K(256, op_rows_on_x<K>(c, false)) MKD_CASE_K(2048, op_rows_on_x<K>(c, false)) } return false;)
MKD_EXEC(exec_lm_head, switch (kp->hidden) { MKD_CASE_K(256, op_rows_on_x<K>(c, true)) MKD_CASE_K(2048, op_rows_on_x<K>(c, true)) } return false;)
MKD_EXEC(exec_oproj, switch (kp->n_q * kp->head_dim / kp->n_kv) { MKD_CASE_K(256, op_oproj<K>(c)) MKD_CASE_K(1024, op_oproj<K>(c)) } return false;)
MKD_EXEC(exec_moe_up, switch (kp->hidden) { MKD_CASE_K(256, op_moe_up<K>(c)) MKD_CASE_K(2048, op_moe_up<K>(c)) } return false;)
MKD_EXEC(exec_moe_down, switch (kp->inter) { MKD_CASE_K(128, op_moe_down<K>(c)) MKD_CASE_K(768, op_moe_down<K>(c)) } return false;)
MKD_EXEC(exec_attn, if (kp->head_dim == 128) return op_attn<128>(c); if (kp->head_dim == 64) return op_attn<64>(c); return false;)

__device__ __forceinline__ bool run_task(KParams* kp, LAS char* lds, const GAS int32_t* d, int32_t task) {
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

// Trace record of a finished task (thread 0; fields in LDS were set by the task).
__device__ __forceinline__ void trace_task(KParams* kp, LAS int32_t* mi, const GAS int32_t* d, uint64_t t0) {
  GAS uint64_t* trace = gas(kp->trace);
  if (trace && threadIdx.x == 0) {
    const int32_t gi = d[D_GIDX];
    if (gi >= 0 && gi < kp->trace_cap) {
      const uint64_t ready = ((uint64_t)(uint32_t)mi[MI_READY_HI] << 32) | (uint32_t)mi[MI_READY_LO];
      GAS uint64_t* r = trace + (int64_t)gi * 4;
      r[0] = t0;
      r[1] = ready ? ready : t0;
      r[2] = wall_clock64();
      r[3] = (uint64_t)(uint32_t)d[D_OPCODE] | ((uint64_t)blockIdx.x << 16) | ((uint64_t)(uint32_t)mi[MI_ITEMS] << 32);
    }
  }
}

__device__ __forceinline__ void reset_task_state(LAS int32_t* mi, bool first) {
  if (threadIdx.x == 0) {
    if (first) {
      mi[MI_WAIT_CTR] = -1;
      mi[MI_WAIT_TGT] = 0;
    }
    mi[MI_ITEMS] = 0;
    mi[MI_READY_LO] = 0;
    mi[MI_READY_HI] = 0;
  }
  __syncthreads();
}

// Persistent interpreter: workgroup i walks task list i.
__global__ void __launch_bounds__(kThreads, 1) mk_persistent(Params prm) {
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  LAS char* lds = (LAS char*)lds_raw;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  LAS int32_t* mi = reinterpret_cast<LAS int32_t*>(lds + kLdsMisc);
  const GAS int32_t* offs = gas(kp->cu_offsets);
  const int begin = offs[blockIdx.x], end = offs[blockIdx.x + 1];
  for (int t = begin; t < end; ++t) {
    const GAS int32_t* d = gas(kp->tasks) + (int64_t)t * D_WORDS;
    reset_task_state(mi, t == begin);
    const uint64_t t0 = kp->trace ? wall_clock64() : 0;
    const bool ok = run_task(kp, lds, d, t);
    trace_task(kp, mi, d, t0);
    if (!ok) break;
    __syncthreads();
  }
}

// Ablation: one launch per wave of tasks; block i runs task first + i.
__global__ void __launch_bounds__(kThreads, 1) mk_wave(Params prm, int32_t first) {
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  LAS char* lds = (LAS char*)lds_raw;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  LAS int32_t* mi = reinterpret_cast<LAS int32_t*>(lds + kLdsMisc);
  const int32_t t = first + (int32_t)blockIdx.x;
  const GAS int32_t* d = gas(kp->tasks) + (int64_t)t * D_WORDS;
  reset_task_state(mi, true);
  const uint64_t t0 = kp->trace ? wall_clock64() : 0;
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
