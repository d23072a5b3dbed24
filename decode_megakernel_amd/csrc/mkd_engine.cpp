// mkd_engine.cpp - C-ABI of the decode megakernel (declared in include/mkd.h).
//
// Host side of one step ("Inside the megakernel serving engine for North Mini Code",
// section "The serving engine around the kernel": clear per-step state, select the
// schedule, launch the megakernel): validate the arguments, pick the cached plan for
// the batch size, zero the step's counters with a fill kernel, and make one
// cooperative launch of the persistent interpreter (or, in the ablation mode, one
// launch per wave of tasks).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/mkd.h"
#include "mkd_common.h"
#include "mkd_plan.h"

namespace mkd {
hipError_t launch_clear(uint32_t* counters, int32_t n, hipStream_t s);
hipError_t launch_persistent(const Params& p, int n_wg, hipStream_t s);
hipError_t launch_wave(const Params& p, int32_t first, int32_t count, hipStream_t s);
int geometry_index(int hidden, int inter, int hd);
}  // namespace mkd

using namespace mkd;

namespace {

thread_local std::string g_create_error;

struct DevPlan {
  Plan plan;
  int32_t* d_per_cu = nullptr;
  int32_t* d_offsets = nullptr;
  int32_t* d_global = nullptr;
};

}  // namespace

struct mkd_engine {
  mkd_config cfg{};
  Geometry geom{};
  int32_t device = -1;
  int32_t max_batch = 0, max_pages = 0, n_cu = 0;
  PlanOptions opts;
  PlanShape shape{};
  CounterLayout ctr{};
  bool have_weights = false;
  mkd_weights w{};
  int32_t mode = MKD_MODE_MEGAKERNEL;
  // workspace
  void* ws = nullptr;
  size_t ws_bytes = 0;
  Params base{};
  int32_t max_attn_items = 0;
  std::map<int32_t, DevPlan> plans;
  std::string err;
  int32_t last_batch = 0;
  hipStream_t last_stream = nullptr;
  uint64_t* trace = nullptr;
  int32_t trace_cap = 0;
  uint32_t epoch = 0;  // number of the last step, in [1, 2^24) (0: none yet; the workspace starts zeroed)
  std::vector<std::pair<void*, size_t>> tagged;  // workspace buffers of tagged words
  ~mkd_engine() {
    if (device >= 0) {
      hipSetDevice(device);
      for (auto& kv : plans) {
        hipFree(kv.second.d_per_cu);
        hipFree(kv.second.d_offsets);
        hipFree(kv.second.d_global);
      }
      hipFree(ws);
    }
  }
};

namespace {

int fail(mkd_engine* e, int code, const std::string& msg) {
  if (e) e->err = msg;
  return code;
}

int hip_fail(mkd_engine* e, hipError_t rc, const char* what) {
  return fail(e, MKD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(rc));
}

std::string check_config(const mkd_config& c, int32_t max_batch, int32_t max_pages) {
  if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 ||
      c.n_experts < 1 || c.top_k < 1 || c.moe_inter < 1 || c.vocab < 1 || c.page_size < 1)
    return "all dimensions must be positive";
  if (c.n_layers > 254) return "at most 254 layers (tagged words carry the layer in 8 bits)";
  if (c.n_q_heads % c.n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
  if (c.n_q_heads / c.n_kv_heads > 16) return "at most 16 query heads per KV group";
  if (geometry_index(c.hidden, c.moe_inter, c.head_dim) < 0)
    return "(hidden, moe_inter, head_dim) must be (2048, 768, 128) or (256, 128, 64): the kernel is compiled "
           "for these geometries";
  if ((c.n_q_heads * c.head_dim) % c.hidden || (c.n_q_heads * c.head_dim) / c.hidden > 4)
    return "n_q_heads * head_dim must be 1, 2 or 4 times hidden";
  if (c.n_experts > 256) return "at most 256 experts";
  if (c.top_k > 16 || c.top_k > c.n_experts) return "top_k must be <= 16 and <= n_experts";
  if (c.page_size != 16) return "page_size must be 16";
  if (c.n_kv_heads > 16) return "at most 16 KV groups";
  if (!(c.rms_eps >= 0.0f) || !(c.rope_base > 0.0f)) return "rms_eps >= 0 and rope_base > 0 required";
  if (max_batch < 1 || max_batch > 16) return "max_batch must be in [1, 16]";
  if (max_pages < 1) return "max_pages_per_seq must be positive";
  if (max_pages > 24576) return "max_pages_per_seq must be <= 24576 (393216 tokens)";
  return "";
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int mkd_create(const mkd_config* cfg, int32_t hip_device, int32_t max_batch, int32_t max_pages_per_seq,
               mkd_engine** out) {
  if (!out) return MKD_ERR_ARG;
  *out = nullptr;
  if (!cfg) {
    g_create_error = "cfg is NULL";
    return MKD_ERR_ARG;
  }
  const std::string bad = check_config(*cfg, max_batch, max_pages_per_seq);
  if (!bad.empty()) {
    g_create_error = bad;
    return MKD_ERR_ARG;
  }
  std::unique_ptr<mkd_engine> e(new mkd_engine());
  e->cfg = *cfg;
  e->geom = Geometry{cfg->n_layers, cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim,
                     cfg->n_experts, cfg->top_k, cfg->moe_inter, cfg->vocab, cfg->page_size};
  e->max_batch = max_batch;
  e->max_pages = max_pages_per_seq;
  e->shape = make_shape(e->geom, e->opts, 1);
  e->ctr = make_counters(e->geom, e->shape, max_batch);
  {
    const int ppi = std::min(e->opts.pages_per_item, e->opts.pages_per_item_2);
    e->max_attn_items = max_batch * cfg->n_kv_heads * ((max_pages_per_seq + ppi - 1) / ppi);
  }
  if (hip_device < 0) {  // host-only engine: plan inspection
    e->n_cu = 0;
    *out = e.release();
    return MKD_OK;
  }
  hipError_t rc = hipSetDevice(hip_device);
  if (rc != hipSuccess) {
    g_create_error = std::string("hipSetDevice: ") + hipGetErrorString(rc);
    return MKD_ERR_HIP;
  }
  e->device = hip_device;
  hipDeviceProp_t prop;
  rc = hipGetDeviceProperties(&prop, hip_device);
  if (rc != hipSuccess) {
    g_create_error = std::string("hipGetDeviceProperties: ") + hipGetErrorString(rc);
    return MKD_ERR_HIP;
  }
  if (!prop.cooperativeLaunch) {
    g_create_error = "device does not support cooperative launches";
    return MKD_ERR_HIP;
  }
  e->n_cu = prop.multiProcessorCount;
  // workspace layout
  const int64_t L = cfg->n_layers, B = max_batch, H = cfg->hidden, E = cfg->n_experts, K = cfg->top_k;
  const int64_t QD = (int64_t)cfg->n_q_heads * cfg->head_dim, hpg = cfg->n_q_heads / cfg->n_kv_heads;
  Params& p = e->base;
  const size_t part_bytes = sizeof(uint64_t) * (size_t)e->max_attn_items * hpg * (cfg->head_dim + 2);
  const size_t attn_o_bytes = sizeof(uint64_t) * L * B * QD;
  const size_t router_bytes = sizeof(uint64_t) * L * B * E;
  const size_t tbl_bytes = sizeof(uint64_t) * L * kRouteTableWords;
  const size_t act_bytes = sizeof(uint64_t) * L * B * K * cfg->moe_inter;
  const size_t h_bytes = sizeof(uint64_t) * (L + 1) * B * H;
  const size_t q_bytes = sizeof(uint64_t) * L * B * QD;
  const size_t flag_bytes = sizeof(uint64_t) * L * 2 * cfg->n_kv_heads * 64;
  const size_t ss_bytes = sizeof(uint64_t) * (L + 1) * B * e->shape.n_rt;
  const size_t rope_bytes = sizeof(uint64_t) * B * cfg->head_dim;
  std::vector<std::pair<size_t, void**>> slots = {
      {h_bytes, (void**)&p.h},
      {ss_bytes, (void**)&p.ss},
      {q_bytes, (void**)&p.q},
      {flag_bytes, (void**)&p.kvflag},
      {part_bytes, (void**)&p.attn_part},
      {attn_o_bytes, (void**)&p.attn_o},
      {router_bytes, (void**)&p.router},
      {tbl_bytes, (void**)&p.route_tbl},
      {sizeof(int32_t) * L * B * K, (void**)&p.topk_ids},
      {sizeof(float) * L * B * K, (void**)&p.topk_w},
      {act_bytes, (void**)&p.moe_act},
      {sizeof(double) * cfg->head_dim / 2, (void**)&p.inv_freq},
      {rope_bytes, (void**)&p.rope},
      {1024, (void**)&p.dummy},
      {sizeof(uint32_t) * (size_t)e->ctr.total, (void**)&p.counters},
  };
  size_t total = 0;
  for (auto& s : slots) total += align256(s.first);
  rc = hipMalloc(&e->ws, total);
  if (rc != hipSuccess) {
    g_create_error = std::string("hipMalloc workspace: ") + hipGetErrorString(rc);
    return MKD_ERR_HIP;
  }
  e->ws_bytes = total;
  size_t at = 0;
  for (auto& s : slots) {
    *s.second = (char*)e->ws + at;
    at += align256(s.first);
  }
  e->tagged = {{p.attn_part, part_bytes}, {p.attn_o, attn_o_bytes}, {p.router, router_bytes}, {p.route_tbl, tbl_bytes},
               {p.moe_act, act_bytes}, {p.h, h_bytes}, {p.ss, ss_bytes}, {p.rope, rope_bytes},
               {p.q, q_bytes}, {p.kvflag, flag_bytes}};
  rc = hipMemset(e->ws, 0, total);
  if (rc == hipSuccess) {
    std::vector<double> inv(cfg->head_dim / 2);
    for (int i = 0; i < cfg->head_dim / 2; ++i)
      inv[i] = std::pow((double)cfg->rope_base, -2.0 * (double)i / (double)cfg->head_dim);
    rc = hipMemcpy((void*)p.inv_freq, inv.data(), sizeof(double) * inv.size(), hipMemcpyHostToDevice);
  }
  if (rc != hipSuccess) {
    g_create_error = std::string("workspace init: ") + hipGetErrorString(rc);
    return MKD_ERR_HIP;
  }
  p.n_layers = cfg->n_layers;
  p.hidden = cfg->hidden;
  p.n_q = cfg->n_q_heads;
  p.n_kv = cfg->n_kv_heads;
  p.head_dim = cfg->head_dim;
  p.n_experts = cfg->n_experts;
  p.top_k = cfg->top_k;
  p.inter = cfg->moe_inter;
  p.vocab = cfg->vocab;
  p.page = cfg->page_size;
  p.rms_eps = cfg->rms_eps;
  p.max_batch = max_batch;
  p.max_pages = max_pages_per_seq;
  p.shape = e->shape;
  p.ctr = e->ctr;
  p.max_attn_items = e->max_attn_items;
  p.spin_limit = 4000000;
  *out = e.release();
  return MKD_OK;
}

void mkd_destroy(mkd_engine* eng) { delete eng; }

int mkd_load_weights(mkd_engine* e, const mkd_weights* w) {
  if (!e) return MKD_ERR_ARG;
  if (!w || !w->embed || !w->norm || !w->w_qkv || !w->w_o || !w->w_router || !w->w_gate_up || !w->w_down)
    return fail(e, MKD_ERR_ARG, "every weight pointer must be non-NULL");
  e->w = *w;
  e->base.embed = (const uint16_t*)w->embed;
  e->base.norm = (const uint16_t*)w->norm;
  e->base.w_qkv = (const uint16_t*)w->w_qkv;
  e->base.w_o = (const uint16_t*)w->w_o;
  e->base.w_router = (const uint16_t*)w->w_router;
  e->base.w_gate_up = (const uint16_t*)w->w_gate_up;
  e->base.w_down = (const uint16_t*)w->w_down;
  e->have_weights = true;
  return MKD_OK;
}

int mkd_set_mode(mkd_engine* e, int32_t mode) {
  if (!e) return MKD_ERR_ARG;
  if (mode != MKD_MODE_MEGAKERNEL && mode != MKD_MODE_OP_PER_KERNEL) return fail(e, MKD_ERR_ARG, "unknown mode");
  e->mode = mode;
  return MKD_OK;
}

static int get_plan(mkd_engine* e, int32_t batch, DevPlan** out) {
  auto it = e->plans.find(batch);
  if (it != e->plans.end()) {
    *out = &it->second;
    return MKD_OK;
  }
  DevPlan dp;
  const std::string bad = build_plan(e->geom, e->opts, e->max_batch, batch, e->n_cu, &dp.plan);
  if (!bad.empty()) return fail(e, MKD_ERR_ARG, "plan: " + bad);
  hipError_t rc = hipMalloc(&dp.d_per_cu, sizeof(int32_t) * dp.plan.per_cu.size());
  if (rc == hipSuccess) rc = hipMalloc(&dp.d_global, sizeof(int32_t) * dp.plan.global.size());
  if (rc == hipSuccess) rc = hipMalloc(&dp.d_offsets, sizeof(int32_t) * dp.plan.cu_offsets.size());
  if (rc == hipSuccess)
    rc = hipMemcpy(dp.d_per_cu, dp.plan.per_cu.data(), sizeof(int32_t) * dp.plan.per_cu.size(),
                   hipMemcpyHostToDevice);
  if (rc == hipSuccess)
    rc = hipMemcpy(dp.d_global, dp.plan.global.data(), sizeof(int32_t) * dp.plan.global.size(),
                   hipMemcpyHostToDevice);
  if (rc == hipSuccess)
    rc = hipMemcpy(dp.d_offsets, dp.plan.cu_offsets.data(), sizeof(int32_t) * dp.plan.cu_offsets.size(),
                   hipMemcpyHostToDevice);
  if (rc != hipSuccess) {
    hipFree(dp.d_per_cu);
    hipFree(dp.d_global);
    hipFree(dp.d_offsets);
    return hip_fail(e, rc, "plan upload");
  }
  auto ins = e->plans.emplace(batch, dp);
  *out = &ins.first->second;
  return MKD_OK;
}

int mkd_decode_step(mkd_engine* e, void* stream, int32_t batch, const int32_t* d_tokens,
                    const int32_t* d_seq_lens, const int32_t* h_seq_lens, const int32_t* d_page_table,
                    const int32_t* h_page_table, void* kv_pool, int32_t n_pages, float* d_logits) {
  if (!e) return MKD_ERR_ARG;
  if (e->device < 0) return fail(e, MKD_ERR_STATE, "host-only engine cannot decode");
  if (!e->have_weights) return fail(e, MKD_ERR_STATE, "weights not loaded");
  if (batch < 1 || batch > e->max_batch)
    return fail(e, MKD_ERR_CAPACITY, "batch must be in [1, max_batch]");
  if (!d_tokens || !d_seq_lens || !h_seq_lens || !d_page_table || !kv_pool || !d_logits)
    return fail(e, MKD_ERR_ARG, "NULL pointer argument");
  if (n_pages < 1) return fail(e, MKD_ERR_ARG, "n_pages must be positive");
  const int P = e->cfg.page_size;
  hipError_t rc = hipSetDevice(e->device);
  if (rc != hipSuccess) return hip_fail(e, rc, "hipSetDevice");
  DevPlan* dp = nullptr;
  int r = get_plan(e, batch, &dp);
  if (r != MKD_OK) return r;
  // attention items per step: one team takes larger items once the step's items at the
  // plan's size outnumber the CUs (every item costs a claim, a merge and a partial result),
  // and the largest once they outnumber them four times over at that larger size
  int ppi = dp->plan.shape.pages_per_item;
  if (dp->plan.n_teams == 1) {
    auto n_items = [&](int size) {
      int64_t n = 0;
      for (int b = 0; b < batch; ++b)
        n += (int64_t)e->cfg.n_kv_heads * ((std::max(h_seq_lens[b], 0) / P + 1 + size - 1) / size);
      return n;
    };
    if (n_items(ppi) > e->n_cu) {
      ppi = e->opts.pages_per_item_long;
      if (n_items(ppi) > 4 * (int64_t)e->n_cu) ppi = e->opts.pages_per_item_max;
    }
  }
  int64_t items = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t s = h_seq_lens[b];
    if (s < 0) return fail(e, MKD_ERR_ARG, "negative sequence length");
    if (s / P >= e->max_pages)
      return fail(e, MKD_ERR_CAPACITY, "sequence " + std::to_string(b) + " needs more pages than max_pages_per_seq");
    if (h_page_table) {
      for (int lp = 0; lp <= s / P; ++lp) {
        const int32_t pg = h_page_table[(int64_t)b * e->max_pages + lp];
        if (pg < 0 || pg >= n_pages)
          return fail(e, MKD_ERR_ARG, "page table entry (" + std::to_string(b) + ", " + std::to_string(lp) +
                                          ") = " + std::to_string(pg) + " is outside [0, n_pages)");
      }
    }
    items += (int64_t)e->cfg.n_kv_heads * ((s / P + 1 + ppi - 1) / ppi);
  }
  if (items > e->max_attn_items) return fail(e, MKD_ERR_CAPACITY, "attention work exceeds the workspace");
  Params p = e->base;
  p.n_teams = dp->plan.n_teams;
  p.shape = dp->plan.shape;
  p.shape.pages_per_item = ppi;
  p.batch = batch;
  p.n_pages = n_pages;
  p.tokens = d_tokens;
  p.seq_lens = d_seq_lens;
  p.page_table = d_page_table;
  p.kv_pool = (uint16_t*)kv_pool;
  p.logits = d_logits;
  p.cu_offsets = dp->d_offsets;
  p.trace = e->trace;
  p.trace_cap = e->trace_cap;
  // A fresh epoch per step (tagged words carry (epoch << 8) | layer).  Epoch 0 is never
  // used, so zeroed words never read as ready; when the 24-bit epoch wraps, the tagged
  // buffers are cleared first, so no word from 2^24 steps ago can pass for a new one.
  hipStream_t s = (hipStream_t)stream;
  if (++e->epoch >= (1u << 24)) {
    e->epoch = 1;
    for (const auto& t : e->tagged) {
      rc = launch_clear((uint32_t*)t.first, (int32_t)(t.second / 4), s);
      if (rc != hipSuccess) return hip_fail(e, rc, "tag clear");
    }
  }
  p.epoch = e->epoch;
  rc = launch_clear(p.counters, e->ctr.total, s);
  if (rc != hipSuccess) return hip_fail(e, rc, "counter clear");
  if (e->mode == MKD_MODE_MEGAKERNEL) {
    p.tasks = dp->d_per_cu;
    rc = launch_persistent(p, e->n_cu, s);
    if (rc != hipSuccess) return hip_fail(e, rc, "megakernel launch");
  } else {
    p.tasks = dp->d_global;
    for (const Wave& w : dp->plan.waves) {
      if (w.count == 0) continue;
      rc = launch_wave(p, w.first, w.count, s);
      if (rc != hipSuccess) return hip_fail(e, rc, "wave launch");
    }
  }
  e->last_batch = batch;
  e->last_stream = s;
  e->err.clear();
  return MKD_OK;
}

int mkd_sync_status(mkd_engine* e) {
  if (!e) return MKD_ERR_ARG;
  if (e->device < 0) return MKD_OK;
  hipError_t rc = hipSetDevice(e->device);
  if (rc == hipSuccess) rc = hipStreamSynchronize(e->last_stream);
  if (rc != hipSuccess) return hip_fail(e, rc, "stream synchronize");
  uint32_t st[G_COUNT];
  rc = hipMemcpy(st, e->base.counters + e->ctr.global_base, sizeof(st), hipMemcpyDeviceToHost);
  if (rc != hipSuccess) return hip_fail(e, rc, "status read");
  if (st[G_ERR_CODE] == 0) return MKD_OK;
  char buf[256];
  if (st[G_ERR_CODE] == 1 && (int32_t)st[G_ERR_CTR] == G_TAGGED) {
    snprintf(buf, sizeof(buf), "watchdog: task %u waited on tagged data (saw tag %u, wanted %u)", st[G_ERR_TASK],
             st[G_ERR_SEEN], st[G_ERR_WANT]);
    fail(e, MKD_ERR_DEADLOCK, buf);
  } else if (st[G_ERR_CODE] == 1) {
    snprintf(buf, sizeof(buf), "watchdog: task %u waited on counter %u (saw %u, wanted %u)", st[G_ERR_TASK],
             st[G_ERR_CTR], st[G_ERR_SEEN], st[G_ERR_WANT]);
    fail(e, MKD_ERR_DEADLOCK, buf);
  } else {
    snprintf(buf, sizeof(buf), "invalid input on device: task %u saw %d (limit %u)", st[G_ERR_TASK],
             (int)st[G_ERR_SEEN], st[G_ERR_WANT]);
    fail(e, MKD_ERR_ARG, buf);
  }
  const int code = st[G_ERR_CODE] == 1 ? MKD_ERR_DEADLOCK : MKD_ERR_ARG;
  hipMemset(e->base.counters + e->ctr.global_base, 0, sizeof(st));
  return code;
}

int mkd_set_trace(mkd_engine* e, void* dev_buf, size_t bytes) {
  if (!e) return MKD_ERR_ARG;
  if (dev_buf && bytes < 32) return fail(e, MKD_ERR_ARG, "trace buffer smaller than one record");
  e->trace = (uint64_t*)dev_buf;
  e->trace_cap = dev_buf ? (int32_t)std::min<size_t>(bytes / 32, 0x7FFFFFFF) : 0;
  return MKD_OK;
}

const char* mkd_last_error(const mkd_engine* e) { return e ? e->err.c_str() : g_create_error.c_str(); }

int mkd_debug_read(mkd_engine* e, int32_t what, void* dst, size_t bytes) {
  if (!e || !dst) return MKD_ERR_ARG;
  if (e->device < 0) return fail(e, MKD_ERR_STATE, "host-only engine");
  const int64_t B = e->last_batch, L = e->cfg.n_layers, mb = e->max_batch;
  if (B < 1) return fail(e, MKD_ERR_STATE, "no step has run");
  int64_t inner = 0, outer = 0;  // inner: 4-byte values per (layer, token) row
  const char* src = nullptr;
  bool tagged = false;  // the buffer holds tagged words: the value is each word's low half
  switch (what) {
    case MKD_DEBUG_HIDDEN:
      inner = e->cfg.hidden; outer = L + 1; src = (const char*)e->base.h; tagged = true; break;
    case MKD_DEBUG_TOPK_IDS: inner = e->cfg.top_k; outer = L; src = (const char*)e->base.topk_ids; break;
    case MKD_DEBUG_TOPK_W: inner = e->cfg.top_k; outer = L; src = (const char*)e->base.topk_w; break;
    case MKD_DEBUG_ROUTER:
      inner = e->cfg.n_experts; outer = L; src = (const char*)e->base.router; tagged = true; break;
    default: return fail(e, MKD_ERR_ARG, "unknown debug buffer");
  }
  if (bytes < (size_t)(outer * B * inner * 4)) return fail(e, MKD_ERR_ARG, "debug buffer too small");
  hipError_t rc = hipSetDevice(e->device);
  if (rc == hipSuccess) rc = hipStreamSynchronize(e->last_stream);
  // one copy per layer row (a strided 2-D copy was seen to leave the destination
  // untouched under a profiler's interception)
  const int64_t wb = tagged ? 8 : 4;  // bytes per stored word
  std::vector<uint64_t> row(tagged ? (size_t)(B * inner) : 0);
  for (int64_t o = 0; o < outer && rc == hipSuccess; ++o) {
    char* d = (char*)dst + o * B * inner * 4;
    const char* sp = src + o * mb * inner * wb;
    if (!tagged) {
      rc = hipMemcpy(d, sp, (size_t)(B * inner * 4), hipMemcpyDeviceToHost);
    } else {
      rc = hipMemcpy(row.data(), sp, (size_t)(B * inner * 8), hipMemcpyDeviceToHost);
      for (int64_t i = 0; i < B * inner; ++i) {
        const uint32_t v = (uint32_t)row[i];
        std::memcpy(d + i * 4, &v, 4);
      }
    }
  }
  if (rc != hipSuccess) return hip_fail(e, rc, "debug read");
  return MKD_OK;
}

int mkd_plan_inspect(mkd_engine* e, int32_t batch, int32_t n_cu, int32_t* desc, int32_t max_tasks,
                     int32_t* cu_offsets, int32_t* n_tasks, int32_t* n_teams) {
  if (!e || !n_tasks) return MKD_ERR_ARG;
  Plan plan;
  const std::string bad = build_plan(e->geom, e->opts, e->max_batch, batch, n_cu, &plan);
  if (!bad.empty()) return fail(e, MKD_ERR_ARG, "plan: " + bad);
  *n_tasks = plan.n_tasks();
  if (n_teams) *n_teams = plan.n_teams;
  if (plan.n_tasks() > max_tasks) return fail(e, MKD_ERR_CAPACITY, "max_tasks too small");
  if (desc) std::memcpy(desc, plan.per_cu.data(), sizeof(int32_t) * plan.per_cu.size());
  if (cu_offsets) std::memcpy(cu_offsets, plan.cu_offsets.data(), sizeof(int32_t) * plan.cu_offsets.size());
  return MKD_OK;
}

}  // extern "C"
