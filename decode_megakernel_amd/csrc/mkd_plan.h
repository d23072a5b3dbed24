// mkd_plan.h - host task scheduler for the decode megakernel.
//
// "Inside the megakernel serving engine for North Mini Code", section "The task
// scheduler: mapping tasks to SMs": the host builds named waves for each layer,
// chooses an order, flattens them into one task list and deals task k to compute
// unit k mod n_cu; attention and the MoE stages reserve a fixed number of claimer
// tasks that drain shared queues.  Any order without circular waits is correct; the
// order only changes throughput.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "mkd_common.h"

#ifndef MKD_MAXP
#define MKD_MAXP 1  // attention pages per worker wave (kernel register budget)
#endif
#ifndef MKD_UP_ROWS_LARGE
#define MKD_UP_ROWS_LARGE 16
#endif
#ifndef MKD_UP_ROWS_LARGE_FROM
#define MKD_UP_ROWS_LARGE_FROM 2
#endif
#ifndef MKD_UP_ROWS
#define MKD_UP_ROWS 12  // batch 1, 8K context: 4 -> 268, 8 -> 289, 12 -> 293, 16 -> 291 tok/s
#endif
#ifndef MKD_QKV_TPH
#define MKD_QKV_TPH 4  // batch 1, 8K (21-page items): 3 -> 377, 4 -> 381, auto (6) -> 381; with 28-page items 3 -> 396, 4 -> 405, 5 -> 366 tok/s
#endif
#ifndef MKD_PPI
#define MKD_PPI 28  // batch 1, 8K context, 4 QKV tiles per head: 24 -> 388, 28 -> 405, 32 -> 400 tok/s
#endif
#ifndef MKD_ROUTER_ROWS
#define MKD_ROUTER_ROWS 8
#endif
#ifndef MKD_PPI_LONG
#define MKD_PPI_LONG 56  // batch 1, 32K context: 28 -> 257, 42 -> 312, 56 -> 321, 64 -> 311 tok/s
#endif

namespace mkd {

struct Geometry {
  int32_t n_layers, hidden, n_q, n_kv, head_dim, n_experts, top_k, inter, vocab, page;
};

// Wave kinds of one layer, in the order they can be arranged.  W_ATTN_MOE is the merged
// wave of the interleaved order (attention and MoE-up claimers alternating).
enum WaveKind : int32_t { W_QKV = 0, W_ROUTER, W_ATTN, W_MOE_UP, W_MOE_DOWN, W_OUT, W_KINDS, W_ATTN_MOE = W_KINDS };

// Named wave orders ("The task scheduler: mapping tasks to SMs": the default order and
// its two ablations, mapped onto this design's waves, in which the attention combine
// belongs to the attention claimers and the O-proj to the output tasks):
//   ORDER_DEFAULT      qkv -> router -> attention -> MoE-up -> MoE-down -> output
//   ORDER_ATTN_FIRST   qkv -> attention -> router -> MoE-up -> MoE-down -> output (attention
//                      is dealt before any routing or expert work)
//   ORDER_MOE_FIRST    router -> qkv -> MoE-up -> MoE-down -> attention -> output
//   ORDER_INTERLEAVED  qkv -> router -> (attention, MoE-up claimers alternating) -> MoE-down
//                      -> output: dealt round robin, the two branches run side by side on
//                      disjoint CUs
enum ScheduleOrder : int32_t { ORDER_DEFAULT = 0, ORDER_ATTN_FIRST, ORDER_MOE_FIRST, ORDER_INTERLEAVED, ORDER_COUNT };
// Placement of the global order onto workgroups (workgroup w runs on XCD w mod 8):
//   PLACE_ROUND_ROBIN  task k -> workgroup k mod n_cu (consecutive tasks on different XCDs)
//   PLACE_XCD          task k -> the (k mod n_cu)-th slot of an XCD-major numbering, so that
//                      runs of n_cu / 8 consecutive tasks share one XCD and its L2
enum SchedulePlacement : int32_t { PLACE_ROUND_ROBIN = 0, PLACE_XCD, PLACE_COUNT };
constexpr int32_t kXcds = 8;

struct PlanOptions {
  int32_t rt_rows = 8;         // residual rows per output task (O-proj + expert down rows)
  int32_t up_rows = MKD_UP_ROWS;  // activation rows per MoE-up item at most (weights: 2x rows); the
                                  // largest divisor of the expert inter size not above it is used
  // ... for schedules whose batches reach up_rows_large_from: larger items, whose fixed
  // cost (claim, ring start, barriers) weighs less when the items are claimed from the
  // queue (8K context: batch 2 515 -> 522-527 tok/s, 4: 667 -> 689, 8: 748 -> 775, 16:
  // 809 -> 828-833 with 16 rows; batch 1, which streams its items, keeps 12: 430 vs 419)
  int32_t up_rows_large = MKD_UP_ROWS_LARGE;
  int32_t up_rows_large_from = MKD_UP_ROWS_LARGE_FROM;
  int32_t pages_per_item = MKD_PPI;  // attention pages per claimed item (7 worker waves)
  // when the step's attention items at pages_per_item outnumber the CUs (long contexts):
  // larger items, since every item pays a claim, a merge and a partial result; when they
  // still outnumber the CUs four times over (batch 1 at 256K: 56 -> 97, 64 -> 107 tok/s;
  // batch 4 at 64K: 315 -> 320), the largest, pages_per_item_max
  int32_t pages_per_item_long = MKD_PPI_LONG;
  int32_t pages_per_item_max = 64;
  int32_t qkv_max_pairs = 17;  // RoPE pairs per QKV tile at most (tile = 2x rows); a head is
                               // split into about n_cu / heads tiles so that one pass of QKV
                               // tiles covers the compute units once
  int32_t qkv_tph = MKD_QKV_TPH;  // QKV tiles per head when > 0 (tiles of up to 24 pairs): fewer,
                                  // larger tiles leave the CUs after them free for attention
  int32_t router_rows = MKD_ROUTER_ROWS;
  int32_t lm_rows = 32;
  int32_t n_attn_claimers = 0; // 0: automatic
  int32_t n_up_claimers = 0;
  // Order of the waves inside a layer: the pages' default order (qkv -> router ->
  // attention -> MoE -> output), which measured fastest of the orders tried (MoE-up
  // before attention: 25% slower; router before QKV: no change).
  int32_t order[W_KINDS] = {W_QKV, W_ROUTER, W_ATTN, W_MOE_UP, W_MOE_DOWN, W_OUT};
  int32_t down_rows = 64;  // expert down rows per MoE-down item (a divisor of hidden)
  // ... for schedules whose batches reach down_rows_large_from (8K context: batch 8 772 -> 780
  // tok/s, 16: 832 -> 841 with 128 rows; batch 2 and 4 were 1% slower with them)
  int32_t down_rows_large = 128;
  int32_t down_rows_large_from = 8;
  int32_t n_down_claimers = 0;  // 0: one per CU
  int32_t interleave = 0;  // merge the attention and MoE-up waves (ORDER_INTERLEAVED)
  int32_t placement = PLACE_ROUND_ROBIN;
};

// Sets o.order / o.interleave / o.placement for a named schedule; "" or an error.
std::string set_schedule(PlanOptions* o, int32_t order, int32_t placement);

struct Wave {
  int32_t kind;   // WaveKind, or -1 for embed, -2 for LM head
  int32_t layer;
  int32_t first;  // index into the global-order task array
  int32_t count;
};

struct Plan {
  int32_t n_cu = 0;
  PlanShape shape{};
  CounterLayout ctr{};
  std::vector<int32_t> global;      // [n][32] tasks in global (flattened) order
  std::vector<Wave> waves;          // ranges of `global`
  std::vector<int32_t> per_cu;      // [n][32] tasks grouped by CU, each list in global order
  std::vector<int32_t> cu_offsets;  // [n_cu + 1]
  int32_t n_tasks() const { return (int32_t)(global.size() / D_WORDS); }
};

// Shape constants and counter layout (independent of the batch size).
PlanShape make_shape(const Geometry& g, const PlanOptions& o, int32_t max_batch);
CounterLayout make_counters(const Geometry& g);

// Build the schedule for batches of up to `max_batch` sequences on `n_cu` compute units.
// The task lists do not depend on the batch size: the claimers size their work from the
// step's sequence lengths.  Returns "" on success, else a description of the violated
// constraint.
std::string build_plan(const Geometry& g, const PlanOptions& o, int32_t max_batch, int32_t n_cu, Plan* out);

// Static checks of a plan: every tagged edge's producer wave precedes its consumer wave
// in the global order, and every compute unit's list is in increasing global order (so
// no task waits for one placed after it on its own CU and no circular wait exists).
// Returns "" if valid.
std::string validate_plan(const Geometry& g, const Plan& p);

}  // namespace mkd
