// mkd_plan.cpp - host task scheduler (see mkd_plan.h).
#include "mkd_plan.h"

#include <algorithm>
#include <cstring>

namespace mkd {

// MoE-up item rows: the largest divisor of the expert inter size not above the option
// for the schedule's batch size.
static int32_t up_rows_for(const Geometry& g, const PlanOptions& o, int32_t max_batch) {
  const int32_t want = max_batch >= o.up_rows_large_from ? o.up_rows_large : o.up_rows;
  int32_t r = std::max(1, std::min(want, g.inter));
  while (g.inter % r) --r;
  return r;
}

static int32_t down_rows_for(const PlanOptions& o, int32_t max_batch) {
  return max_batch >= o.down_rows_large_from ? o.down_rows_large : o.down_rows;
}

PlanShape make_shape(const Geometry& g, const PlanOptions& o, int32_t max_batch) {
  PlanShape s{};
  s.rt_rows = o.rt_rows;
  s.n_rt = g.hidden / o.rt_rows;
  s.up_rows = up_rows_for(g, o, max_batch);
  s.n_up_tiles = g.inter / s.up_rows;
  s.pages_per_item = o.pages_per_item;
  s.qkv_rows = 2 * o.qkv_max_pairs;
  s.router_rows = o.router_rows;
  s.lm_rows = o.lm_rows;
  s.down_rows = down_rows_for(o, max_batch);
  s.n_down_chunks = g.hidden / s.down_rows;
  return s;
}

CounterLayout make_counters(const Geometry& g) {
  CounterLayout c{};
  int32_t at = 0;
  c.attn_claim = at++;
  c.up_claim = at++;
  c.down_claim = at++;
  c.per_layer = (at + 15) / 16 * 16;
  c.global_base = c.per_layer * (g.n_layers + 1);
  c.total = c.global_base + G_COUNT;
  return c;
}

namespace {

struct Emitter {
  std::vector<int32_t>* v;
  int32_t wave_id = 0;
  int32_t emit(int32_t op, int32_t layer, int32_t a0, int32_t a1, int32_t a2, int32_t a3) {
    const size_t at = v->size();
    v->resize(at + D_WORDS, 0);
    int32_t* d = v->data() + at;
    d[D_OPCODE] = op;
    d[D_LAYER] = layer;
    d[D_ARG0] = a0;
    d[D_ARG1] = a1;
    d[D_ARG2] = a2;
    d[D_ARG3] = a3;
    d[D_WAVE] = wave_id;
    d[D_GIDX] = (int32_t)(at / D_WORDS);
    return d[D_GIDX];
  }
};

}  // namespace

std::string set_schedule(PlanOptions* o, int32_t order, int32_t placement) {
  static const int32_t orders[ORDER_COUNT][W_KINDS] = {
      {W_QKV, W_ROUTER, W_ATTN, W_MOE_UP, W_MOE_DOWN, W_OUT},
      {W_QKV, W_ATTN, W_ROUTER, W_MOE_UP, W_MOE_DOWN, W_OUT},
      {W_ROUTER, W_QKV, W_MOE_UP, W_MOE_DOWN, W_ATTN, W_OUT},
      {W_QKV, W_ROUTER, W_ATTN, W_MOE_UP, W_MOE_DOWN, W_OUT},
  };
  if (order < 0 || order >= ORDER_COUNT) return "unknown schedule order";
  if (placement < 0 || placement >= PLACE_COUNT) return "unknown placement";
  for (int i = 0; i < W_KINDS; ++i) o->order[i] = orders[order][i];
  o->interleave = order == ORDER_INTERLEAVED ? 1 : 0;
  o->placement = placement;
  return "";
}

std::string build_plan(const Geometry& g, const PlanOptions& o, int32_t max_batch, int32_t n_cu, Plan* out) {
  if (max_batch < 1 || max_batch > 16) return "max_batch must be in [1, 16]";
  if (n_cu < 1) return "n_cu must be positive";
  if (g.hidden % o.rt_rows) return "hidden must be a multiple of rt_rows";
  if (o.rt_rows & (o.rt_rows - 1)) return "rt_rows must be a power of two";
  if (g.hidden / o.rt_rows > 256) return "hidden / rt_rows must be at most 256";
  if ((g.n_q * g.head_dim) % g.hidden || (g.n_q * g.head_dim) / g.hidden > 4)
    return "n_q * head_dim must be 1, 2 or 4 times hidden";
  if (o.rt_rows * ((g.n_q * g.head_dim) / g.hidden) > 35 || 4 * o.rt_rows > 35)
    return "output tiles are limited to 35 GEMV rows";
  if (o.up_rows < 1) return "up_rows must be positive";
  if (o.qkv_max_pairs < 1) return "qkv_max_pairs must be positive";
  // the output task keeps each lane's (row, token) residual words in registers: 2 per lane
  if (o.rt_rows * max_batch > 128) return "rt_rows * max_batch must be at most 128";
  if (g.n_experts > 256) return "at most 256 experts";
  if (o.pages_per_item < 1 || o.pages_per_item > 64) return "pages_per_item must be in [1, 64]";
  if (o.pages_per_item_long < o.pages_per_item || o.pages_per_item_max < o.pages_per_item_long ||
      o.pages_per_item_max > 64)
    return "pages_per_item <= pages_per_item_long <= pages_per_item_max <= 64 is required";
  // a GEMV tile holds at most 5 row steps per worker wave (7 workers, >= 1 row per step)
  if (o.rt_rows > 35 || 2 * std::max(o.up_rows, o.up_rows_large) > 35 || 2 * o.qkv_max_pairs > 35 || o.router_rows > 35 || o.lm_rows > 35)
    return "GEMV tiles are limited to 35 rows";
  {
    // a MoE-down item is one GEMV tile over rows of length inter whose row sums (one per
    // row and token of its expert) fit the 2048-float row-sum area
    const int dr = down_rows_for(o, max_batch);
    if (dr < 1 || g.hidden % dr || dr * max_batch > 2048)
      return "MoE-down rows must divide hidden, with rows * max_batch <= 2048";
  }
  Plan& P = *out;
  P = Plan();
  P.n_cu = n_cu;
  P.shape = make_shape(g, o, max_batch);
  P.ctr = make_counters(g);
  const PlanShape& s = P.shape;
  const CounterLayout& c = P.ctr;
  auto L = [&](int l, int off) { return l * c.per_layer + off; };
  Emitter em{&P.global};
  auto begin_wave = [&](int32_t kind, int32_t layer) {
    P.waves.push_back(Wave{kind, layer, P.n_tasks(), 0});
    em.wave_id = (int32_t)P.waves.size() - 1;
  };
  auto end_wave = [&]() { P.waves.back().count = P.n_tasks() - P.waves.back().first; };

  const int n_qkv_heads = g.n_q + 2 * g.n_kv;
  const int half = g.head_dim / 2;
  // tiles per head: about n_cu / heads, within [ceil(half / max_pairs), half]; the pairs of
  // a head are split as evenly as possible
  const int qkv_tph = o.qkv_tph > 0 ? std::min(half, std::max(o.qkv_tph, (half + 23) / 24))
                                    : std::min(half, std::max((half + o.qkv_max_pairs - 1) / o.qkv_max_pairs,
                                                              n_cu / n_qkv_heads));
  if (2 * ((half + qkv_tph - 1) / qkv_tph) * max_batch > 2048) return "QKV tile rows x batch exceed the row-sum area";
  if (qkv_tph > 64) return "at most 64 QKV tiles per head";
  P.shape.qkv_tph = qkv_tph;
  const int n_router_tiles = (g.n_experts + o.router_rows - 1) / o.router_rows;
  const int n_attn = o.n_attn_claimers > 0 ? o.n_attn_claimers : n_cu;
  const int n_up = o.n_up_claimers > 0 ? o.n_up_claimers : n_cu;
  // no MoE-down claimers when no batch of this schedule reaches the split (their tasks
  // would only cost a dispatch on every CU per layer)
  const int n_down = max_batch < kDownSplitBatch ? 0 : o.n_down_claimers > 0 ? o.n_down_claimers : n_cu;

  begin_wave(-1, 0);
  // residual rows, their sums of squares and the RoPE table leave as tagged words
  for (int rt = 0; rt < s.n_rt; ++rt) em.emit(OP_EMBED, 0, rt, 0, 0, 0);
  end_wave();
  for (int l = 0; l < g.n_layers; ++l) {
    for (int wi = 0; wi < W_KINDS; ++wi) {
      const int kind = o.order[wi];
      if (o.interleave && kind == W_MOE_UP) continue;  // merged into the attention wave
      if (o.interleave && kind == W_ATTN) {
        // claimer i of each queue at global positions 2i and 2i + 1
        begin_wave(W_ATTN_MOE, l);
        for (int i = 0; i < std::max(n_attn, n_up); ++i) {
          if (i < n_attn) em.emit(OP_ATTN, l, i, n_attn, 0, 0);
          if (i < n_up) em.emit(OP_MOE_UP, l, i, n_up, 0, 0);
        }
        end_wave();
        continue;
      }
      begin_wave(kind, l);
      switch (kind) {
        case W_QKV:
          for (int hh = 0; hh < n_qkv_heads; ++hh)
            for (int t = 0; t < qkv_tph; ++t) {
              const int j0 = t * half / qkv_tph, j1 = (t + 1) * half / qkv_tph;
              // queries leave tagged; K / V tiles raise a tagged flag (ARG3: tile of the head)
              em.emit(OP_QKV, l, hh, j0, j1 - j0, t);
            }
          break;
        case W_ROUTER:
          for (int r0 = 0; r0 < g.n_experts; r0 += o.router_rows)
            // logits leave as tagged words (no counter): consumers wait on the data itself
            // ARG2 = 1: the first tile also builds and publishes the layer's routing tables
            em.emit(OP_ROUTER, l, r0, std::min(o.router_rows, g.n_experts - r0), r0 == 0 ? 1 : 0, 0);
          break;
        case W_ATTN:
          for (int i = 0; i < n_attn; ++i)
            em.emit(OP_ATTN, l, i, n_attn, 0, 0);
          break;
        case W_MOE_UP:
          for (int i = 0; i < n_up; ++i)
            em.emit(OP_MOE_UP, l, i, n_up, 0, 0);
          break;
        case W_MOE_DOWN:
          for (int i = 0; i < n_down; ++i)
            em.emit(OP_MOE_DOWN, l, i, n_down, 0, 0);
          break;
        case W_OUT:
          // waits inside the task: the combined attention of every KV group, then the up
          // tiles of every active expert (dynamic: routing decides the experts)
          for (int rt = 0; rt < s.n_rt; ++rt) em.emit(OP_OUT, l, rt, 0, 0, 0);
          break;
        default:
          return "bad wave order";
      }
      end_wave();
    }
  }
  begin_wave(-2, g.n_layers);
  for (int r0 = 0; r0 < g.vocab; r0 += o.lm_rows)
    em.emit(OP_LM_HEAD, g.n_layers, r0, std::min(o.lm_rows, g.vocab - r0), 0, 0);
  end_wave();

  // Deal the tasks round robin, keeping global order within each list: task k goes to
  // workgroup k mod n_cu, or with XCD placement to the workgroup of XCD-major slot
  // k mod n_cu (slot q: XCD q / (n_cu / 8), workgroup (q mod (n_cu / 8)) * 8 + XCD).
  const int n = P.n_tasks();
  const int n_lists = n_cu;
  const bool xcd = o.placement == PLACE_XCD && n_cu % kXcds == 0;
  if (o.placement == PLACE_XCD && !xcd) return "XCD placement needs a multiple of 8 compute units";
  const int per_xcd = n_cu / kXcds;
  std::vector<std::vector<int32_t>> lists(n_lists);
  for (int k = 0; k < n; ++k) {
    const int q = k % n_cu;
    lists[xcd ? (q % per_xcd) * kXcds + q / per_xcd : q].push_back(k);
  }
  P.cu_offsets.assign(n_lists + 1, 0);
  P.per_cu.reserve(P.global.size());
  for (int li = 0; li < n_lists; ++li) {
    P.cu_offsets[li] = (int32_t)(P.per_cu.size() / D_WORDS);
    for (int32_t k : lists[li])
      P.per_cu.insert(P.per_cu.end(), P.global.begin() + (size_t)k * D_WORDS,
                      P.global.begin() + (size_t)(k + 1) * D_WORDS);
  }
  P.cu_offsets[n_lists] = (int32_t)(P.per_cu.size() / D_WORDS);
  return validate_plan(g, P);
}

std::string validate_plan(const Geometry& g, const Plan& P) {
  const int n = P.n_tasks();
  // Every descriptor is well formed; the reserved words are zero.
  for (int k = 0; k < n; ++k) {
    const int32_t* d = P.global.data() + (size_t)k * D_WORDS;
    if (d[D_GIDX] != k) return "task " + std::to_string(k) + ": global index mismatch";
    const int op = d[D_OPCODE];
    if (op < OP_NOP || op >= OP_COUNT) return "task " + std::to_string(k) + ": bad opcode";
    for (int w = D_GIDX + 1; w < D_WORDS; ++w)
      if (d[w] != 0) return "task " + std::to_string(k) + ": reserved descriptor word set";
  }
  // Edges carried by tagged data (no counter): the router logits (MoE-up claimers and
  // output tasks read them), the attention partials and combined output (output tasks),
  // and the experts' activations (output tasks).  Their producers' waves precede their
  // consumers' waves in the global order.
  for (int l = 0; l < g.n_layers; ++l) {
    int router_end = -1, up_first = -1, attn_end = -1, up_end = -1, out_first = -1, qkv_end = -1, attn_first = -1;
    int down_first = -1, down_end = -1;
    for (const Wave& w : P.waves)
      if (w.layer == l) {
        if (w.kind == W_ROUTER) router_end = w.first + w.count;
        if (w.kind == W_QKV) qkv_end = w.first + w.count;
        if (w.kind == W_ATTN) attn_first = w.first;
        if (w.kind == W_ATTN) attn_end = w.first + w.count;
        if (w.kind == W_MOE_UP) {
          up_first = w.first;
          up_end = w.first + w.count;
        }
        if (w.kind == W_ATTN_MOE) {
          attn_first = up_first = w.first;
          attn_end = up_end = w.first + w.count;
        }
        if (w.kind == W_MOE_DOWN) {
          down_first = w.first;
          down_end = w.first + w.count;
        }
        if (w.kind == W_OUT) out_first = w.first;
      }
    if (qkv_end < 0 || attn_first < qkv_end)
      return "layer " + std::to_string(l) + ": the attention wave must follow the QKV wave";
    if (router_end < 0 || up_first < router_end)
      return "layer " + std::to_string(l) + ": the MoE-up wave must follow the router wave";
    // the layer's input: the previous layer's output wave (the embedding wave for layer 0)
    // precedes every task of the layer
    int prev_end = -1, first = -1;
    for (const Wave& w : P.waves) {
      if ((l == 0 && w.kind == -1) || (l > 0 && w.layer == l - 1 && w.kind == W_OUT)) prev_end = w.first + w.count;
      if (w.layer == l && w.kind >= 0 && (first < 0 || w.first < first)) first = w.first;
    }
    if (prev_end < 0 || first < prev_end)
      return "layer " + std::to_string(l) + ": its tasks must follow the previous layer's output wave";
    if (down_first < 0 || down_first < up_end)
      return "layer " + std::to_string(l) + ": the MoE-down wave must follow the MoE-up wave";
    if (attn_end < 0 || up_end < 0 || out_first < 0 || out_first < attn_end || out_first < up_end ||
        out_first < down_end)
      return "layer " + std::to_string(l) + ": the output wave must follow the attention and MoE waves";
  }
  {
    int last_out_end = -1, lm_first = -1;
    for (const Wave& w : P.waves) {
      if (w.layer == g.n_layers - 1 && w.kind == W_OUT) last_out_end = w.first + w.count;
      if (w.kind == -2 && w.count > 0) lm_first = w.first;
    }
    if (lm_first >= 0 && lm_first < last_out_end) return "the LM-head wave must follow the last output wave";
  }
  // every list in increasing global order, every task in exactly one list
  if ((int)P.cu_offsets.size() != P.n_cu + 1) return "wrong number of task lists";
  std::vector<char> seen(n, 0);
  for (int li = 0; li + 1 < (int)P.cu_offsets.size(); ++li) {
    int32_t prev = -1;
    for (int t = P.cu_offsets[li]; t < P.cu_offsets[li + 1]; ++t) {
      const int32_t gi = P.per_cu[(size_t)t * D_WORDS + D_GIDX];
      if (gi <= prev) return "list " + std::to_string(li) + ": not in global order";
      if (gi < 0 || gi >= n || seen[gi]) return "task " + std::to_string(gi) + " listed twice or out of range";
      seen[gi] = 1;
      prev = gi;
    }
  }
  for (int k = 0; k < n; ++k)
    if (!seen[k]) return "task " + std::to_string(k) + " is in no list";
  return "";
}

}  // namespace mkd
