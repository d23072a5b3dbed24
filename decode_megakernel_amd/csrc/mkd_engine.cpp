// mkd_engine.cpp - C-ABI of the decode megakernel (declared in include/mkd.h).
//
// Host side of one step ("Inside the megakernel serving engine for North Mini Code",
// section "The serving engine around the kernel": clear per-step state, select the
// schedule, launch the megakernel): validate the arguments, choose the step's attention
// item size, zero the step's counters with a fill kernel, and make one cooperative launch
// of the persistent interpreter (or, in the ablation mode, one launch per wave of tasks).
// The schedule is built once per engine (section "The task scheduler: mapping tasks to
// SMs") and copied into the caller's workspace when the workspace is handed over, so a
// step allocates nothing and copies nothing synchronously.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <string>
#include <vector>

#include "../../include/mkd.h"
#include "mkd_common.h"
#include "mkd_plan.h"

namespace mkd {
hipError_t launch_clear(uint32_t* words, int64_t n, hipStream_t s);
hipError_t launch_persistent(const Params& p, int n_wg, hipStream_t s);
hipError_t launch_wave(const Params& p, int32_t first, int32_t count, hipStream_t s);
int geometry_index(int hidden, int inter, int hd);
}  // namespace mkd

using namespace mkd;

namespace {

thread_local std::string g_create_error;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// One region of the workspace: byte offset from the workspace start, size, and whether it
// holds tagged words (cleared again when the step epoch wraps).
struct Region {
  size_t off = 0, bytes = 0;
  bool tagged = false;
};

}  // namespace

struct mkd_engine {
  uint64_t id = 0;  // distinct for every engine created in the process
  mkd_config cfg{};
  Geometry geom{};
  int32_t device = -1;
  int32_t max_batch = 0, max_pages = 0, n_cu = 0;
  PlanOptions opts;
  Plan plan;  // built in mkd_create (device engines)
  bool have_weights = false;
  int32_t mode = MKD_MODE_MEGAKERNEL;
  // workspace layout (offsets) and the caller's buffer
  Region r_h, r_ss, r_q, r_kvflag, r_part, r_attn_o, r_router, r_tbl, r_topk_ids, r_topk_w, r_act, r_moe_part,
      r_inv_freq, r_rope, r_dummy, r_counters, r_tasks_cu, r_tasks_global, r_offsets;
  size_t ws_bytes = 0;
  char* ws = nullptr;
  Params base{};
  int32_t max_attn_items = 0;
  std::string err;
  int32_t last_batch = 0;
  hipStream_t last_stream = nullptr;
  char* last_ws = nullptr;  // workspace of the last step (the engine's or the static scratch)
  uint64_t* trace = nullptr;
  int32_t trace_cap = 0;
  int32_t spin_limit = 4000000;
  int32_t attn_window = 0, full_every = 1;  // local-attention layers (mkd_set_attention_window)
  uint32_t epoch = 0;  // number of the last step, in [1, 2^24) (0: none since the workspace was cleared)
  std::vector<double> inv_freq;  // RoPE frequencies base^(-2i/hd), copied into every workspace
  std::vector<const Region*> regions() const {
    return {&r_h, &r_ss, &r_q, &r_kvflag, &r_part, &r_attn_o, &r_router, &r_tbl, &r_topk_ids,
            &r_topk_w, &r_act, &r_moe_part, &r_inv_freq, &r_rope, &r_dummy, &r_counters, &r_tasks_cu,
            &r_tasks_global, &r_offsets};
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

// Workspace layout of an engine (offsets only; the plan must be built).
void layout(mkd_engine* e) {
  const mkd_config& c = e->cfg;
  const int64_t L = c.n_layers, B = e->max_batch, H = c.hidden, E = c.n_experts, K = c.top_k;
  const int64_t QD = (int64_t)c.n_q_heads * c.head_dim, hpg = c.n_q_heads / c.n_kv_heads;
  const int64_t n_rt = e->plan.shape.n_rt;
  size_t at = 0;
  auto put = [&](Region& r, size_t bytes, bool tagged) {
    r.off = at;
    r.bytes = bytes;
    r.tagged = tagged;
    at += align256(bytes);
  };
  const size_t w8 = sizeof(uint64_t);
  put(e->r_h, w8 * (L + 1) * B * H, true);
  put(e->r_ss, w8 * (L + 1) * B * n_rt, true);
  put(e->r_q, w8 * L * B * QD, true);
  put(e->r_kvflag, w8 * L * 2 * c.n_kv_heads * 64, true);
  put(e->r_part, w8 * (size_t)e->max_attn_items * hpg * (c.head_dim + 2), true);
  put(e->r_attn_o, w8 * L * B * QD, true);
  put(e->r_router, w8 * L * B * E, true);
  put(e->r_tbl, w8 * L * kRouteTableWords, true);
  put(e->r_topk_ids, sizeof(int32_t) * L * B * K, false);
  put(e->r_topk_w, sizeof(float) * L * B * K, false);
  put(e->r_act, w8 * L * B * K * c.moe_inter, true);
  // one layer's expert output rows per (token, choice); every layer reuses it (its tags
  // carry the layer)
  put(e->r_moe_part, w8 * B * K * H, true);
  put(e->r_inv_freq, sizeof(double) * c.head_dim / 2, false);
  put(e->r_rope, w8 * B * c.head_dim, true);
  put(e->r_dummy, 1024, false);
  put(e->r_counters, sizeof(uint32_t) * (size_t)e->plan.ctr.total, false);
  put(e->r_tasks_cu, sizeof(int32_t) * e->plan.per_cu.size(), false);
  put(e->r_tasks_global, sizeof(int32_t) * e->plan.global.size(), false);
  put(e->r_offsets, sizeof(int32_t) * e->plan.cu_offsets.size(), false);
  e->ws_bytes = at;
}

// Workspace pointers of the kernel parameters for a workspace starting at `ws`.
void point_params(const mkd_engine* e, char* ws, Params& p) {
  p.h = (uint64_t*)(ws + e->r_h.off);
  p.ss = (uint64_t*)(ws + e->r_ss.off);
  p.q = (uint64_t*)(ws + e->r_q.off);
  p.kvflag = (uint64_t*)(ws + e->r_kvflag.off);
  p.attn_part = (uint64_t*)(ws + e->r_part.off);
  p.attn_o = (uint64_t*)(ws + e->r_attn_o.off);
  p.router = (uint64_t*)(ws + e->r_router.off);
  p.route_tbl = (uint64_t*)(ws + e->r_tbl.off);
  p.topk_ids = (int32_t*)(ws + e->r_topk_ids.off);
  p.topk_w = (float*)(ws + e->r_topk_w.off);
  p.moe_act = (uint64_t*)(ws + e->r_act.off);
  p.moe_part = (uint64_t*)(ws + e->r_moe_part.off);
  p.inv_freq = (const double*)(ws + e->r_inv_freq.off);
  p.rope = (uint64_t*)(ws + e->r_rope.off);
  p.dummy = ws + e->r_dummy.off;
  p.counters = (uint32_t*)(ws + e->r_counters.off);
}

uint64_t g_next_engine_id = 1;

}  // namespace

namespace mkd {

// Clear a workspace at `ws` and copy the schedule and the RoPE frequencies into it, in
// order on `stream` (every tagged word then carries epoch 0, which no step uses).
hipError_t init_workspace(const mkd_engine* e, char* ws, hipStream_t stream) {
  hipError_t rc = launch_clear((uint32_t*)ws, (int64_t)(e->ws_bytes / 4), stream);
  const Plan& P = e->plan;
  if (rc == hipSuccess)
    rc = hipMemcpyAsync(ws + e->r_inv_freq.off, e->inv_freq.data(), sizeof(double) * e->inv_freq.size(),
                        hipMemcpyHostToDevice, stream);
  if (rc == hipSuccess)
    rc = hipMemcpyAsync(ws + e->r_tasks_cu.off, P.per_cu.data(), sizeof(int32_t) * P.per_cu.size(),
                        hipMemcpyHostToDevice, stream);
  if (rc == hipSuccess)
    rc = hipMemcpyAsync(ws + e->r_tasks_global.off, P.global.data(), sizeof(int32_t) * P.global.size(),
                        hipMemcpyHostToDevice, stream);
  if (rc == hipSuccess)
    rc = hipMemcpyAsync(ws + e->r_offsets.off, P.cu_offsets.data(), sizeof(int32_t) * P.cu_offsets.size(),
                        hipMemcpyHostToDevice, stream);
  // the sources are the engine's own vectors, which outlive the copies
  return rc;
}

}  // namespace mkd

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
  e->id = g_next_engine_id++;
  e->cfg = *cfg;
  e->geom = Geometry{cfg->n_layers, cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim,
                     cfg->n_experts, cfg->top_k, cfg->moe_inter, cfg->vocab, cfg->page_size};
  e->max_batch = max_batch;
  e->max_pages = max_pages_per_seq;
  for (int i = 0; i < cfg->head_dim / 2; ++i)
    e->inv_freq.push_back(std::pow((double)cfg->rope_base, -2.0 * (double)i / (double)cfg->head_dim));
  e->max_attn_items = max_batch * cfg->n_kv_heads * ((max_pages_per_seq + e->opts.pages_per_item - 1) /
                                                     e->opts.pages_per_item);
  if (hip_device < 0) {  // host-only engine: plan inspection
    *out = e.release();
    return MKD_OK;
  }
  hipDeviceProp_t prop;
  hipError_t rc = hipGetDeviceProperties(&prop, hip_device);
  if (rc != hipSuccess) {
    g_create_error = std::string("hipGetDeviceProperties: ") + hipGetErrorString(rc);
    return MKD_ERR_HIP;
  }
  if (!prop.cooperativeLaunch) {
    g_create_error = "device does not support cooperative launches";
    return MKD_ERR_HIP;
  }
  e->device = hip_device;
  e->n_cu = prop.multiProcessorCount;
  const std::string pbad = build_plan(e->geom, e->opts, max_batch, e->n_cu, &e->plan);
  if (!pbad.empty()) {
    g_create_error = "plan: " + pbad;
    return MKD_ERR_ARG;
  }
  layout(e.get());
  Params& p = e->base;
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
  p.shape = e->plan.shape;
  p.ctr = e->plan.ctr;
  p.max_attn_items = e->max_attn_items;
  *out = e.release();
  return MKD_OK;
}

void mkd_destroy(mkd_engine* eng) { delete eng; }

size_t mkd_workspace_bytes(const mkd_engine* e) { return (e && e->device >= 0) ? e->ws_bytes : 0; }

int mkd_set_workspace(mkd_engine* e, void* dev_ptr, size_t bytes) {
  if (!e) return MKD_ERR_ARG;
  if (e->device < 0) return fail(e, MKD_ERR_STATE, "host-only engine has no workspace");
  if (!dev_ptr) return fail(e, MKD_ERR_ARG, "workspace pointer is NULL");
  if ((uintptr_t)dev_ptr & 255) return fail(e, MKD_ERR_ARG, "workspace must be 256-byte aligned");
  if (bytes < e->ws_bytes)
    return fail(e, MKD_ERR_ARG, "workspace of " + std::to_string(bytes) + " bytes is smaller than the " +
                                    std::to_string(e->ws_bytes) + " bytes mkd_workspace_bytes asks for");
  hipError_t rc = hipSetDevice(e->device);
  if (rc != hipSuccess) return hip_fail(e, rc, "hipSetDevice");
  e->ws = nullptr;
  rc = init_workspace(e, (char*)dev_ptr, nullptr);
  if (rc == hipSuccess) rc = hipStreamSynchronize(nullptr);
  if (rc != hipSuccess) return hip_fail(e, rc, "workspace initialisation");
  e->ws = (char*)dev_ptr;
  point_params(e, e->ws, e->base);
  e->epoch = 0;
  e->last_batch = 0;
  e->last_ws = nullptr;
  return MKD_OK;
}

int mkd_set_schedule(mkd_engine* e, int32_t order, int32_t placement) {
  if (!e) return MKD_ERR_ARG;
  PlanOptions o = e->opts;
  const std::string bad = set_schedule(&o, order, placement);
  if (!bad.empty()) return fail(e, MKD_ERR_ARG, bad);
  if (e->device >= 0) {
    Plan plan;
    const std::string pbad = build_plan(e->geom, o, e->max_batch, e->n_cu, &plan);
    if (!pbad.empty()) return fail(e, MKD_ERR_ARG, "plan: " + pbad);
    // the same number of tasks and waves: the workspace layout does not change
    if (plan.per_cu.size() != e->plan.per_cu.size() || plan.global.size() != e->plan.global.size())
      return fail(e, MKD_ERR_STATE, "schedule changed the task count");
    e->plan = std::move(plan);
    if (e->ws) {
      hipError_t rc = hipSetDevice(e->device);
      if (rc == hipSuccess) rc = init_workspace(e, e->ws, nullptr);
      if (rc == hipSuccess) rc = hipStreamSynchronize(nullptr);
      if (rc != hipSuccess) return hip_fail(e, rc, "schedule upload");
      e->epoch = 0;
      e->last_batch = 0;
      e->last_ws = nullptr;
    }
  }
  e->opts = o;
  return MKD_OK;
}

int mkd_load_weights(mkd_engine* e, const mkd_weights* w) {
  if (!e) return MKD_ERR_ARG;
  if (!w || !w->embed || !w->norm || !w->w_qkv || !w->w_o || !w->w_router || !w->w_gate_up || !w->w_down)
    return fail(e, MKD_ERR_ARG, "every weight pointer must be non-NULL");
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

int mkd_set_attention_window(mkd_engine* e, int32_t window, int32_t full_every) {
  if (!e) return MKD_ERR_ARG;
  if (window < 0 || full_every < 1) return fail(e, MKD_ERR_ARG, "window must be >= 0 and full_every >= 1");
  e->attn_window = window;
  e->full_every = full_every;
  return MKD_OK;
}

int mkd_set_watchdog(mkd_engine* e, int32_t polls) {
  if (!e) return MKD_ERR_ARG;
  if (polls < 1) return fail(e, MKD_ERR_ARG, "the watchdog bound must be at least one poll");
  e->spin_limit = polls;
  return MKD_OK;
}

}  // extern "C"

namespace mkd {

uint64_t engine_id(const mkd_engine* e) { return e->id; }
int32_t engine_device(const mkd_engine* e) { return e->device; }
size_t engine_ws_bytes(const mkd_engine* e) { return e->ws_bytes; }
int engine_fail(mkd_engine* e, int code, const char* msg) { return fail(e, code, msg); }
void engine_limits(const mkd_engine* e, int32_t* max_batch, int32_t* max_pages, int32_t* vocab, int32_t* page) {
  *max_batch = e->max_batch;
  *max_pages = e->max_pages;
  *vocab = e->cfg.vocab;
  *page = e->cfg.page_size;
}

// One step on the workspace at `ws` whose last step used epoch *epoch (advanced here):
// validation, the step's attention item size, the counter clear and the launch.  Shared
// by mkd_decode_step (the caller's workspace) and mkd_decode_step_static.
int enqueue_step(mkd_engine* e, char* ws, uint32_t* epoch, void* stream, int32_t batch, const int32_t* d_tokens,
                 const int32_t* d_seq_lens, const int32_t* h_seq_lens, const int32_t* d_page_table,
                 const int32_t* h_page_table, void* kv_pool, int32_t n_pages, float* d_logits) {
  if (batch < 1 || batch > e->max_batch)
    return fail(e, MKD_ERR_CAPACITY, "batch must be in [1, max_batch]");
  if (!d_tokens || !d_seq_lens || !h_seq_lens || !d_page_table || !kv_pool || !d_logits)
    return fail(e, MKD_ERR_ARG, "NULL pointer argument");
  if (n_pages < 1) return fail(e, MKD_ERR_ARG, "n_pages must be positive");
  const int P = e->cfg.page_size;
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
  }
  // Attention items per step: larger items once the step's items at the plan's size
  // outnumber the CUs (every item costs a claim, a merge and a partial result), and the
  // largest once they outnumber them four times over at that larger size.
  auto n_items = [&](int size) {
    int64_t n = 0;
    for (int b = 0; b < batch; ++b) n += (int64_t)e->cfg.n_kv_heads * ((h_seq_lens[b] / P + 1 + size - 1) / size);
    return n;
  };
  int ppi = e->plan.shape.pages_per_item;
  if (n_items(ppi) > e->n_cu) {
    ppi = e->opts.pages_per_item_long;
    if (n_items(ppi) > 4 * (int64_t)e->n_cu) ppi = e->opts.pages_per_item_max;
  }
  if (n_items(ppi) > e->max_attn_items) return fail(e, MKD_ERR_CAPACITY, "attention work exceeds the workspace");
  hipError_t rc = hipSetDevice(e->device);
  if (rc != hipSuccess) return hip_fail(e, rc, "hipSetDevice");
  Params p = e->base;
  point_params(e, ws, p);
  p.shape.pages_per_item = ppi;
  p.batch = batch;
  p.n_pages = n_pages;
  p.tokens = d_tokens;
  p.seq_lens = d_seq_lens;
  p.page_table = d_page_table;
  p.kv_pool = (uint16_t*)kv_pool;
  p.logits = d_logits;
  p.cu_offsets = (const int32_t*)(ws + e->r_offsets.off);
  p.trace = e->trace;
  p.trace_cap = e->trace_cap;
  p.spin_limit = e->spin_limit;
  p.attn_window = e->attn_window;
  p.full_every = e->full_every;
  // A fresh epoch per step (tagged words carry (epoch << 8) | layer).  Epoch 0 is never
  // used, so zeroed words never read as ready; when the 24-bit epoch wraps, the tagged
  // buffers are cleared first, so no word from 2^24 steps ago can pass for a new one.
  hipStream_t s = (hipStream_t)stream;
  if (++*epoch >= (1u << 24)) {
    *epoch = 1;
    for (const Region* r : e->regions()) {
      if (!r->tagged) continue;
      rc = launch_clear((uint32_t*)(ws + r->off), (int64_t)(r->bytes / 4), s);
      if (rc != hipSuccess) return hip_fail(e, rc, "tag clear");
    }
  }
  p.epoch = *epoch;
  rc = launch_clear(p.counters, e->plan.ctr.total, s);
  if (rc != hipSuccess) return hip_fail(e, rc, "counter clear");
  if (e->mode == MKD_MODE_MEGAKERNEL) {
    p.tasks = (const int32_t*)(ws + e->r_tasks_cu.off);
    rc = launch_persistent(p, e->n_cu, s);
    if (rc != hipSuccess) return hip_fail(e, rc, "megakernel launch");
  } else {
    p.tasks = (const int32_t*)(ws + e->r_tasks_global.off);
    for (const Wave& w : e->plan.waves) {
      if (w.count == 0) continue;
      rc = launch_wave(p, w.first, w.count, s);
      if (rc != hipSuccess) return hip_fail(e, rc, "wave launch");
    }
  }
  e->last_batch = batch;
  e->last_stream = s;
  e->last_ws = ws;
  e->err.clear();
  return MKD_OK;
}

// Checks shared by both step entry points before the workspace is known.
int check_step_state(mkd_engine* e) {
  if (e->device < 0) return fail(e, MKD_ERR_STATE, "host-only engine cannot decode");
  if (!e->have_weights) return fail(e, MKD_ERR_STATE, "weights not loaded");
  return MKD_OK;
}

}  // namespace mkd

extern "C" {

int mkd_decode_step(mkd_engine* e, void* stream, int32_t batch, const int32_t* d_tokens,
                    const int32_t* d_seq_lens, const int32_t* h_seq_lens, const int32_t* d_page_table,
                    const int32_t* h_page_table, void* kv_pool, int32_t n_pages, float* d_logits) {
  if (!e) return MKD_ERR_ARG;
  const int st = check_step_state(e);
  if (st != MKD_OK) return st;
  if (!e->ws) return fail(e, MKD_ERR_STATE, "no workspace: call mkd_set_workspace first");
  return enqueue_step(e, e->ws, &e->epoch, stream, batch, d_tokens, d_seq_lens, h_seq_lens, d_page_table,
                      h_page_table, kv_pool, n_pages, d_logits);
}

int mkd_sync_status(mkd_engine* e) {
  if (!e) return MKD_ERR_ARG;
  if (e->device < 0 || !e->last_ws) return MKD_OK;
  hipError_t rc = hipSetDevice(e->device);
  if (rc == hipSuccess) rc = hipStreamSynchronize(e->last_stream);
  if (rc != hipSuccess) return hip_fail(e, rc, "stream synchronize");
  uint32_t* gblock = (uint32_t*)(e->last_ws + e->r_counters.off) + e->plan.ctr.global_base;
  uint32_t st[G_COUNT];
  rc = hipMemcpy(st, gblock, sizeof(st), hipMemcpyDeviceToHost);
  if (rc != hipSuccess) return hip_fail(e, rc, "status read");
  if (st[G_ERR_CODE] == 0) return MKD_OK;
  char buf[256];
  if (st[G_ERR_CODE] == 1) {
    snprintf(buf, sizeof(buf), "watchdog: task %u waited on tagged data (saw tag %u, wanted %u)", st[G_ERR_TASK],
             st[G_ERR_SEEN], st[G_ERR_WANT]);
    fail(e, MKD_ERR_DEADLOCK, buf);
  } else {
    snprintf(buf, sizeof(buf), "invalid input on device: task %u saw %d (limit %u)", st[G_ERR_TASK],
             (int)st[G_ERR_SEEN], st[G_ERR_WANT]);
    fail(e, MKD_ERR_ARG, buf);
  }
  const int code = st[G_ERR_CODE] == 1 ? MKD_ERR_DEADLOCK : MKD_ERR_ARG;
  std::memset(st, 0, sizeof(st));
  hipMemcpy(gblock, st, sizeof(st), hipMemcpyHostToDevice);
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
  if (e->device < 0 || !e->ws) return fail(e, MKD_ERR_STATE, "no workspace");
  if (e->last_ws != e->ws) return fail(e, MKD_ERR_STATE, "the last step did not run on the engine's workspace");
  const int64_t B = e->last_batch, L = e->cfg.n_layers, mb = e->max_batch;
  const int64_t QD = (int64_t)e->cfg.n_q_heads * e->cfg.head_dim;
  if (B < 1) return fail(e, MKD_ERR_STATE, "no step has run");
  // rows: `outer` blocks of `rows` rows of `inner` 4-byte values; consecutive blocks are
  // `stride` rows apart in the workspace
  int64_t inner = 0, outer = 0, rows = B, stride = mb;
  const Region* r = nullptr;
  switch (what) {
    case MKD_DEBUG_HIDDEN: inner = e->cfg.hidden; outer = L + 1; r = &e->r_h; break;
    case MKD_DEBUG_TOPK_IDS: inner = e->cfg.top_k; outer = L; r = &e->r_topk_ids; break;
    case MKD_DEBUG_TOPK_W: inner = e->cfg.top_k; outer = L; r = &e->r_topk_w; break;
    case MKD_DEBUG_ROUTER: inner = e->cfg.n_experts; outer = L; r = &e->r_router; break;
    case MKD_DEBUG_Q: inner = QD; outer = L; r = &e->r_q; break;
    case MKD_DEBUG_ATTN: inner = QD; outer = L; r = &e->r_attn_o; break;
    case MKD_DEBUG_ROUTE: inner = kRouteTableWords; outer = L; rows = 1; stride = 1; r = &e->r_tbl; break;
    case MKD_DEBUG_ACT:
      inner = e->cfg.moe_inter; outer = L; rows = B * e->cfg.top_k; stride = mb * e->cfg.top_k; r = &e->r_act;
      break;
    default: return fail(e, MKD_ERR_ARG, "unknown debug buffer");
  }
  if (bytes < (size_t)(outer * rows * inner * 4)) return fail(e, MKD_ERR_ARG, "debug buffer too small");
  hipError_t rc = hipSetDevice(e->device);
  if (rc == hipSuccess) rc = hipStreamSynchronize(e->last_stream);
  // one copy per block (a strided 2-D copy was seen to leave the destination untouched
  // under a profiler's interception); tagged words keep the value in their low half
  const int64_t wb = r->tagged ? 8 : 4;
  std::vector<uint64_t> row(r->tagged ? (size_t)(rows * inner) : 0);
  for (int64_t o = 0; o < outer && rc == hipSuccess; ++o) {
    char* d = (char*)dst + o * rows * inner * 4;
    const char* sp = e->ws + r->off + o * stride * inner * wb;
    if (!r->tagged) {
      rc = hipMemcpy(d, sp, (size_t)(rows * inner * 4), hipMemcpyDeviceToHost);
    } else {
      rc = hipMemcpy(row.data(), sp, (size_t)(rows * inner * 8), hipMemcpyDeviceToHost);
      for (int64_t i = 0; i < rows * inner; ++i) {
        const uint32_t v = (uint32_t)row[i];
        std::memcpy(d + i * 4, &v, 4);
      }
    }
  }
  if (rc != hipSuccess) return hip_fail(e, rc, "debug read");
  return MKD_OK;
}

int mkd_plan_inspect(mkd_engine* e, int32_t n_cu, int32_t* desc, int32_t max_tasks, int32_t* cu_offsets,
                     int32_t* n_tasks) {
  if (!e || !n_tasks) return MKD_ERR_ARG;
  Plan plan;
  const std::string bad = build_plan(e->geom, e->opts, e->max_batch, n_cu, &plan);
  if (!bad.empty()) return fail(e, MKD_ERR_ARG, "plan: " + bad);
  *n_tasks = plan.n_tasks();
  if (plan.n_tasks() > max_tasks) return fail(e, MKD_ERR_CAPACITY, "max_tasks too small");
  if (desc) std::memcpy(desc, plan.per_cu.data(), sizeof(int32_t) * plan.per_cu.size());
  if (cu_offsets) std::memcpy(cu_offsets, plan.cu_offsets.data(), sizeof(int32_t) * plan.cu_offsets.size());
  return MKD_OK;
}

}  // extern "C"
