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

struct Smem {
  float* xs;
  float* rowsum;
  int32_t* route;
  int32_t* mi;  // misc ints
  float* mf;    // misc floats (inverse RMS per token)
  __device__ explicit Smem(char* base)
      : xs(reinterpret_cast<float*>(base + kLdsXs)),
        rowsum(reinterpret_cast<float*>(base + kLdsRowsum)),
        route(reinterpret_cast<int32_t*>(base + kLdsRoute)),
        mi(reinterpret_cast<int32_t*>(base + kLdsMisc)),
        mf(reinterpret_cast<float*>(base + kLdsMisc + 512)) {}
};
// misc int slots
constexpr int MI_BCAST = 0;
constexpr int MI_OK = 1;
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
  const Params& p;
  Smem s;
  const int32_t* d;  // descriptor
  int32_t task;      // global task index
  int32_t wait_ctr;  // last satisfied wait of this workgroup (skip repeats)
  uint32_t wait_target;
};

__device__ __forceinline__ uint32_t* layer_ctr(const Params& p, int l, int off) {
  return p.counters + (int64_t)l * p.ctr.per_layer + off;
}

// Spin until counter >= target (thread 0 polls, then acquire; whole workgroup
// returns together).  Returns false when the step is aborted (watchdog).
__device__ bool mk_wait(Ctx& c, uint32_t* ctr, uint32_t target) {
  const int32_t idx = (int32_t)(ctr - c.p.counters);
  if (idx == c.wait_ctr && target <= c.wait_target) return true;
  if (threadIdx.x == 0) {
    int ok = 1;
    int32_t spins = 0;
    uint32_t v;
    while ((v = ctr_load(ctr)) < target) {
      if ((spins & 63) == 63 && aborted(c.p)) { ok = 0; break; }
      if (++spins > c.p.spin_limit) {
        report_error(c.p, 1u, c.task, idx, v, target);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    fence_acquire_agent();
    c.s.mi[MI_OK] = ok;
  }
  __syncthreads();
  const bool ok = c.s.mi[MI_OK] != 0;
  if (ok) {
    c.wait_ctr = idx;
    c.wait_target = target;
  }
  return ok;
}

// Publish this workgroup's stores and add one to the counter; returns the old value.
__device__ uint32_t mk_arrive(Ctx& c, uint32_t* ctr) {
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
__device__ int32_t mk_claim(Ctx& c, uint32_t* head) {
  __syncthreads();
  if (threadIdx.x == 0) c.s.mi[MI_BCAST] = (int32_t)ctr_add(head, 1u);
  __syncthreads();
  return c.s.mi[MI_BCAST];
}

// ------------------------------------------------------------------ GEMV tile
// Weight rows of a tile come from up to two row segments (gate|up, or the two
// halves of a RoPE head) with a common leading dimension.
struct RowSrc {
  const uint16_t* base1;
  const uint16_t* base2;
  int64_t ld;
  int32_t n1;
  __device__ const uint16_t* row(int i) const {
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
__device__ __forceinline__ void gemv_compute(const u32x4 (&wb)[kWreg], const float* xs,
                                             const int32_t* tok, int nb, int R, float* rowsum) {
  using G = Gemv<K>;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int si = 0; si < G::MAXS; ++si) {
    const int row = (w + kWaves * si) * G::RPS + lane / G::LPR;
    if ((w + kWaves * si) * G::RPS >= R) break;  // wave-uniform
    for (int j = 0; j < nb; ++j) {
      const float* x = xs + (int64_t)tok[j] * K;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < G::CPL; ++c) {
        const int kc = lane % G::LPR + G::LPR * c;
        const float4* xp = reinterpret_cast<const float4*>(x + kc * 8);
        acc += dot8(wb[si * G::CPL + c], xp[0], xp[1]);
      }
      acc = group_sum<G::LPR>(acc);
      if (lane % G::LPR == 0 && row < R) rowsum[row * nb + j] = acc;
    }
  }
}

// ------------------------------------------------------------------ activation staging
// inverse RMS of the residual rows h_l[b] from the per-row-tile sums of squares.
__device__ void stage_inv_rms(Ctx& c, int l) {
  const Params& p = c.p;
  if (threadIdx.x < p.batch) {
    const float* ss = p.ss + ((int64_t)l * p.max_batch + threadIdx.x) * p.shape.n_rt;
    float t = 0.0f;
    for (int r = 0; r < p.shape.n_rt; ++r) t += ss[r];
    c.s.mf[threadIdx.x] = 1.0f / sqrtf(t / (float)p.hidden + p.rms_eps);
  }
  __syncthreads();
}

// xs[b][k] = h_l[b][k] * inv_rms[b] * gamma_l[k] for every token of the batch
// (the RMSNorm every consumer of layer l's input applies on the fly).
__device__ void stage_x_normed(Ctx& c, int l) {
  const Params& p = c.p;
  stage_inv_rms(c, l);
  const int H = p.hidden;
  const uint16_t* gamma = p.norm + (int64_t)l * H;
  const int n8 = p.batch * (H / 8);
  for (int i = threadIdx.x; i < n8; i += kThreads) {
    const int b = i / (H / 8), k8 = (i % (H / 8)) * 8;
    const float* hp = p.h + ((int64_t)l * p.max_batch + b) * H + k8;
    const float4 h0 = *reinterpret_cast<const float4*>(hp);
    const float4 h1 = *reinterpret_cast<const float4*>(hp + 4);
    const uint4 gw = *reinterpret_cast<const uint4*>(gamma + k8);
    const float r = c.s.mf[b];
    float4 o0, o1;
    o0.x = h0.x * r * bf_lo(gw.x); o0.y = h0.y * r * bf_hi(gw.x);
    o0.z = h0.z * r * bf_lo(gw.y); o0.w = h0.w * r * bf_hi(gw.y);
    o1.x = h1.x * r * bf_lo(gw.z); o1.y = h1.y * r * bf_hi(gw.z);
    o1.z = h1.z * r * bf_lo(gw.w); o1.w = h1.w * r * bf_hi(gw.w);
    float* xo = c.s.xs + (int64_t)b * H + k8;
    *reinterpret_cast<float4*>(xo) = o0;
    *reinterpret_cast<float4*>(xo + 4) = o1;
  }
  if (threadIdx.x < 16) c.s.mi[MI_TOK + threadIdx.x] = threadIdx.x;
  __syncthreads();
}

// ------------------------------------------------------------------ residual finalisation
// The fused residual add + RMSNorm at the end of a layer ("Where the speedup comes
// from": parallel layers are rejoined only by it).  The last arriver of residual
// row tile rt writes h_{l+1} = h_l + sum_g a_g + sum_ds m_ds for those rows and
// their sum of squares; consumers of layer l+1 normalise on the fly.
__device__ bool finalize_rows(Ctx& c, int l, int rt) {
  const Params& p = c.p;
  fence_acquire_agent();
  const int R = p.shape.rt_rows, H = p.hidden, B = p.batch;
  const int r0 = rt * R;
  float* red = c.s.rowsum;  // [B][R] squares
  for (int i = threadIdx.x; i < B * R; i += kThreads) {
    const int b = i / R, r = r0 + i % R;
    const int64_t hb = (int64_t)b * H + r;
    float v = p.h[(int64_t)l * p.max_batch * H + hb];
    for (int g = 0; g < p.n_kv; ++g) v += p.a_part[(((int64_t)l * p.n_kv + g) * p.max_batch) * H + hb];
    for (int ds = 0; ds < p.shape.n_ds; ++ds)
      v += p.m_part[(((int64_t)l * p.shape.n_ds + ds) * p.max_batch) * H + hb];
    p.h[(int64_t)(l + 1) * p.max_batch * H + hb] = v;
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
__device__ bool arrive_rt(Ctx& c, int l, int rt) {
  const Params& p = c.p;
  const uint32_t old = mk_arrive(c, layer_ctr(p, l, p.ctr.rt + rt));
  if (old + 1 == (uint32_t)(p.n_kv + p.shape.n_ds)) return finalize_rows(c, l, rt);
  return true;
}

// ------------------------------------------------------------------ OP_EMBED
__device__ bool op_embed(Ctx& c) {
  const Params& p = c.p;
  const int rt = c.d[D_ARG0];
  const int R = p.shape.rt_rows, H = p.hidden, B = p.batch;
  float* red = c.s.rowsum;
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
__device__ bool op_qkv(Ctx& c) {
  const Params& p = c.p;
  const int l = c.d[D_LAYER], hh = c.d[D_ARG0], j0 = c.d[D_ARG1], PB = c.d[D_ARG2];
  const int hd = p.head_dim, half = hd / 2, H = p.hidden;
  const uint16_t* wl = p.w_qkv + (int64_t)l * (p.n_q + 2 * p.n_kv) * hd * H;
  const RowSrc src{wl + ((int64_t)hh * hd + j0) * H, wl + ((int64_t)hh * hd + half + j0) * H, H, PB};
  u32x4 wb[kWreg];
  gemv_load<K>(wb, src, 2 * PB);
  if (!mk_wait(c, c.p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
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
      float* q = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * hd + (int64_t)hh * hd;
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
      uint16_t* base = p.kv_pool + pg * (int64_t)p.page * hd;
      if (is_k) {
        base[(int64_t)t * hd + dim] = f32_to_bf16(o1);
        base[(int64_t)t * hd + dim + half] = f32_to_bf16(o2);
      } else {
        base[(int64_t)dim * p.page + t] = f32_to_bf16(o1);
        base[(int64_t)(dim + half) * p.page + t] = f32_to_bf16(o2);
      }
    }
  }
  mk_arrive(c, c.p.counters + c.d[D_SIGNAL]);
  return true;
}

// ------------------------------------------------------------------ OP_ROUTER / OP_LM_HEAD
// Plain GEMV tiles on the normed input: router logits (layer l) or vocabulary logits
// (final norm, tied embedding).
template <int K>
__device__ bool op_rows_on_x(Ctx& c, bool lm_head) {
  const Params& p = c.p;
  const int l = c.d[D_LAYER], r0 = c.d[D_ARG0], R = c.d[D_ARG1];
  const int H = p.hidden;
  const uint16_t* base = lm_head ? p.embed + (int64_t)r0 * H
                                 : p.w_router + ((int64_t)l * p.n_experts + r0) * H;
  const RowSrc src{base, base, H, R};
  u32x4 wb[kWreg];
  gemv_load<K>(wb, src, R);
  if (!mk_wait(c, c.p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  stage_x_normed(c, l);
  const int B = p.batch;
  gemv_compute<K>(wb, c.s.xs, c.s.mi + MI_TOK, B, R, c.s.rowsum);
  __syncthreads();
  for (int i = threadIdx.x; i < R * B; i += kThreads) {
    const int r = i / B, b = i % B;
    if (lm_head) p.logits[(int64_t)b * p.vocab + r0 + r] = c.s.rowsum[i];
    else p.router[((int64_t)l * p.max_batch + b) * p.n_experts + r0 + r] = c.s.rowsum[i];
  }
  if (c.d[D_SIGNAL] >= 0) mk_arrive(c, c.p.counters + c.d[D_SIGNAL]);
  return true;
}

// ------------------------------------------------------------------ OP_OPROJ
// Split-K over KV groups (Figure 7: O-proj for a KV group starts as soon as that
// group's attention output lands): rows [rt*R, +R) of W_o, columns of group g.
template <int K>
__device__ bool op_oproj(Ctx& c) {
  const Params& p = c.p;
  const int l = c.d[D_LAYER], rt = c.d[D_ARG0], g = c.d[D_ARG1];
  const int R = p.shape.rt_rows, H = p.hidden, KO = p.n_q * p.head_dim;
  const uint16_t* base = p.w_o + ((int64_t)l * H + (int64_t)rt * R) * KO + (int64_t)g * K;
  const RowSrc src{base, base, KO, R};
  u32x4 wb[kWreg];
  gemv_load<K>(wb, src, R);
  if (!mk_wait(c, c.p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  const int B = p.batch;
  for (int i = threadIdx.x; i < B * (K / 4); i += kThreads) {
    const int b = i / (K / 4), k4 = (i % (K / 4)) * 4;
    *reinterpret_cast<float4*>(c.s.xs + (int64_t)b * K + k4) =
        *reinterpret_cast<const float4*>(p.attn_o + ((int64_t)l * p.max_batch + b) * KO +
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
__device__ int block_exscan(int v, int32_t* tmp, int& total) {
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
__device__ bool route_layer(Ctx& c, int l, bool write_debug) {
  const Params& p = c.p;
  const int B = p.batch, E = p.n_experts, k = p.top_k;
  int32_t* rt = c.s.route;
  float* rw = reinterpret_cast<float*>(rt + RT_W);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = w; b < B; b += kWaves) {
    const float* r = p.router + ((int64_t)l * p.max_batch + b) * E;
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
__device__ bool op_moe_up(Ctx& c) {
  const Params& p = c.p;
  const int l = c.d[D_LAYER];
  if (!mk_wait(c, c.p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  route_layer(c, l, c.d[D_ARG0] == 0);
  stage_x_normed(c, l);
  const int32_t* rt = c.s.route;
  const int n_act = rt[RT_NACT];
  const int UR = p.shape.up_rows, NT = p.shape.n_up_tiles, H = p.hidden, I = p.inter;
  const int k = p.top_k;
  uint32_t* head = layer_ctr(p, l, p.ctr.up_claim);
  for (;;) {
    const int idx = mk_claim(c, head);
    if (idx >= n_act * NT) break;
    const int a = idx / NT, tile = idx % NT;
    const int e = rt[RT_ACT + a];
    const uint16_t* base = p.w_gate_up + (((int64_t)l * p.n_experts + e) * 2 * I + (int64_t)tile * UR) * H;
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
__device__ bool op_moe_down(Ctx& c) {
  const Params& p = c.p;
  const int l = c.d[D_LAYER];
  if (!mk_wait(c, c.p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
  route_layer(c, l, false);
  const int32_t* rt = c.s.route;
  const float* rw = reinterpret_cast<const float*>(rt + RT_W);
  const int n_act = rt[RT_NACT];
  const int R = p.shape.rt_rows, NDS = p.shape.n_ds, H = p.hidden, I = p.inter, B = p.batch;
  const int k = p.top_k;
  float* macc = c.s.rowsum + 1024;  // [R][B]
  uint32_t* head = layer_ctr(p, l, p.ctr.down_claim);
  for (;;) {
    const int idx = mk_claim(c, head);
    if (idx >= p.shape.n_rt * NDS) break;
    const int rtile = idx / NDS, ds = idx % NDS;
    for (int i = threadIdx.x; i < R * B; i += kThreads) macc[i] = 0.0f;
    for (int a = ds; a < n_act; a += NDS) {
      const int e = rt[RT_ACT + a];
      const uint16_t* base = p.w_down + (((int64_t)l * p.n_experts + e) * H + (int64_t)rtile * R) * I;
      const RowSrc src{base, base, I, R};
      u32x4 wb[kWreg];
      gemv_load<K>(wb, src, R);
      if (!mk_wait(c, layer_ctr(p, l, p.ctr.up_done + e), (uint32_t)p.shape.n_up_tiles)) return false;
      const int o0 = rt[RT_OFF + a], n_e = rt[RT_OFF + a + 1] - o0;
      for (int i = threadIdx.x; i < n_e * (K / 4); i += kThreads) {
        const int j = i / (K / 4), k4 = (i % (K / 4)) * 4;
        const int slot = rt[RT_FLAT + o0 + j];
        *reinterpret_cast<float4*>(c.s.xs + (int64_t)j * K + k4) =
            *reinterpret_cast<const float4*>(p.moe_act + ((int64_t)l * p.max_batch * k + slot) * I + k4);
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
__device__ bool attn_item(Ctx& c, int l, int idx, bool& waited) {
  const Params& p = c.p;
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
    if (!mk_wait(c, c.p.counters + c.d[D_WAIT], (uint32_t)c.d[D_TARGET])) return false;
    waited = true;
  }
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    if (lp[i] < c1 && lp[i] == last) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        kr[i][kk] = *reinterpret_cast<const u32x4*>(p.kv_pool + kbase[i] + (lane & 15) * HD + kk * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int dt = 0; dt < NV; ++dt)
        vr[i][dt] = *reinterpret_cast<const u32x2*>(p.kv_pool + vbase[i] + (dt * 16 + (lane & 15)) * 16 + (lane >> 4) * 4);
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
      const float* qp = p.q + ((int64_t)l * p.max_batch + b) * p.n_q * HD +
                        (int64_t)(g * hpg + head) * HD + kk * 32 + (lane >> 4) * 8;
      const float4 a0 = *reinterpret_cast<const float4*>(qp);
      const float4 a1 = *reinterpret_cast<const float4*>(qp + 4);
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
  float* mw = c.s.xs;
  float* lw = c.s.xs + kWaves * 16;
  float* ow = c.s.xs + 2 * kWaves * 16;
  if (lane < 16) {
    mw[w * 16 + lane] = m;
    lw[w * 16 + lane] = lsum;
  }
  if (head < hpg) {
#pragma unroll
    for (int dt = 0; dt < NV; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ow[((int64_t)w * hpg + head) * HD + dt * 16 + (lane >> 4) * 4 + r] = o[dt][r];
  }
  __syncthreads();
  // merge the waves: unnormalised o, running max m and sum l per head
  float* part = p.attn_part + (int64_t)idx * hpg * (HD + 2);
  for (int t = threadIdx.x; t < hpg * HD; t += kThreads) {
    const int h = t / HD, dd = t % HD;
    float M = -INFINITY;
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mw[ww * 16 + h]);
    float acc = 0.0f, L = 0.0f;
    for (int ww = 0; ww < kWaves; ++ww) {
      const float sc = exp2f(mw[ww * 16 + h] - M);
      acc += sc * ow[((int64_t)ww * hpg + h) * HD + dd];
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
    // last item of (b, g): combine all chunks in order (log-sum-exp merge)
    fence_acquire_agent();
    for (int t = threadIdx.x; t < hpg * HD; t += kThreads) {
      const int h = t / HD, dd = t % HD;
      float M = -INFINITY;
      for (int ci = 0; ci < nchunks; ++ci)
        M = fmaxf(M, p.attn_part[((int64_t)(base_bg + ci) * hpg + h) * (HD + 2) + HD]);
      float num = 0.0f, den = 0.0f;
      for (int ci = 0; ci < nchunks; ++ci) {
        const float* pc = p.attn_part + ((int64_t)(base_bg + ci) * hpg + h) * (HD + 2);
        const float sc = exp2f(pc[HD] - M);
        num += sc * pc[dd];
        den += sc * pc[HD + 1];
      }
      p.attn_o[((int64_t)l * p.max_batch + b) * p.n_q * HD + (int64_t)(g * hpg + h) * HD + dd] = num / den;
    }
    mk_arrive(c, layer_ctr(p, l, p.ctr.comb + g));
  }
  return true;
}

template <int HD>
__device__ bool op_attn(Ctx& c) {
  const Params& p = c.p;
  const int l = c.d[D_LAYER];
  int n_items = 0;
  for (int b = 0; b < p.batch; ++b)
    n_items += ((p.seq_lens[b] / p.page + 1 + p.shape.pages_per_item - 1) / p.shape.pages_per_item) * p.n_kv;
  if (n_items > p.max_attn_items) n_items = p.max_attn_items;
  uint32_t* head = layer_ctr(p, l, p.ctr.attn_claim);
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
#define MKD_CASE_K(KV, CALL) \
  case KV: {                 \
    constexpr int K = KV;    \
    return CALL;             \
  }

__device__ bool run_task(Ctx& c) {
  const Params& p = c.p;
  switch (c.d[D_OPCODE]) {
    case OP_EMBED:
      return op_embed(c);
    case OP_QKV:
      switch (p.hidden) { MKD_CASE_K(256, op_qkv<K>(c)) MKD_CASE_K(512, op_qkv<K>(c)) MKD_CASE_K(1024, op_qkv<K>(c)) MKD_CASE_K(2048, op_qkv<K>(c)) }
      return false;
    case OP_ROUTER:
      switch (p.hidden) { MKD_CASE_K(256, op_rows_on_x<K>(c, false)) MKD_CASE_K(512, op_rows_on_x<K>(c, false)) MKD_CASE_K(1024, op_rows_on_x<K>(c, false)) MKD_CASE_K(2048, op_rows_on_x<K>(c, false)) }
      return false;
    case OP_LM_HEAD:
      switch (p.hidden) { MKD_CASE_K(256, op_rows_on_x<K>(c, true)) MKD_CASE_K(512, op_rows_on_x<K>(c, true)) MKD_CASE_K(1024, op_rows_on_x<K>(c, true)) MKD_CASE_K(2048, op_rows_on_x<K>(c, true)) }
      return false;
    case OP_OPROJ:
      switch (p.n_q * p.head_dim / p.n_kv) { MKD_CASE_K(256, op_oproj<K>(c)) MKD_CASE_K(512, op_oproj<K>(c)) MKD_CASE_K(1024, op_oproj<K>(c)) }
      return false;
    case OP_MOE_UP:
      switch (p.hidden) { MKD_CASE_K(256, op_moe_up<K>(c)) MKD_CASE_K(512, op_moe_up<K>(c)) MKD_CASE_K(1024, op_moe_up<K>(c)) MKD_CASE_K(2048, op_moe_up<K>(c)) }
      return false;
    case OP_MOE_DOWN:
      switch (p.inter) { MKD_CASE_K(128, op_moe_down<K>(c)) MKD_CASE_K(256, op_moe_down<K>(c)) MKD_CASE_K(512, op_moe_down<K>(c)) MKD_CASE_K(768, op_moe_down<K>(c)) }
      return false;
    case OP_ATTN:
      if (p.head_dim == 128) return op_attn<128>(c);
      if (p.head_dim == 64) return op_attn<64>(c);
      return false;
    default:
      return true;
  }
}

// Persistent interpreter: workgroup i walks task list i.
__global__ void __launch_bounds__(kThreads, 1) mk_persistent(Params p) {
  __shared__ __align__(16) char lds[kLdsBytes];
  Ctx c{p, Smem(lds), nullptr, 0, -1, 0};
  const int begin = p.cu_offsets[blockIdx.x], end = p.cu_offsets[blockIdx.x + 1];
  for (int t = begin; t < end; ++t) {
    c.d = p.tasks + (int64_t)t * D_WORDS;
    c.task = t;
    if (!run_task(c)) break;
    __syncthreads();
  }
}

// Ablation: one launch per wave of tasks; block i runs task first + i.
__global__ void __launch_bounds__(kThreads, 1) mk_wave(Params p, int32_t first) {
  __shared__ __align__(16) char lds[kLdsBytes];
  Ctx c{p, Smem(lds), nullptr, 0, -1, 0};
  c.task = first + (int32_t)blockIdx.x;
  c.d = p.tasks + (int64_t)c.task * D_WORDS;
  run_task(c);
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
