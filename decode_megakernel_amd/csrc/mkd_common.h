// mkd_common.h - definitions shared by the host scheduler and the device interpreter:
// the task descriptor, the opcodes, the counter layout and the kernel parameters.
//
// Method: "Inside the megakernel serving engine for North Mini Code", sections
// "Tasks" (sixteen opcodes cover the step; every GEMM opcode shares one body),
// "The task descriptor" (32 int32 fields, field 0 the opcode, then layer, tile,
// split, the barrier to wait on, the count to wait for and the barrier to signal)
// and "Barriers" (counters in global memory, zeroed before each step).
#pragma once
#include <stdint.h>

namespace mkd {

// ---------------------------------------------------------------- opcodes
// Our opcode set.  The pages' sixteen opcodes map onto these as follows:
//   QKV_PROJ            -> OP_QKV (RoPE and the paged-KV append in the epilogue)
//   ROUTER_GEMM         -> OP_ROUTER
//   ROUTER_TOPK, ROUTE_FINALIZE, MOE_GATHER
//                       -> built once per layer by the first OP_ROUTER tile after the
//                          layer's logits are in, published as one tagged table that
//                          every MoE-up claimer and output task copies into its LDS
//   ATTN_DRAIN + ATTN_DECODE -> OP_ATTN (claims (seq, kv group, page chunk) items)
//   ATTN_COMBINE        -> the tail of OP_ATTN: after its claim loop, claimer i merges
//                          the chunks of the query heads (b, h) with (b*nq + h) mod
//                          n_claimers == i, from the items' tagged partials
//   MOE_UPGATE_ACT_DRAIN -> OP_MOE_UP
//   MOE_DOWN_DRAIN      -> at batch >= kDownSplitBatch, OP_MOE_DOWN: claimed (active expert,
//                          chunk of down rows) items, each leaving the expert's output rows
//                          for each of its tokens as tagged partials; below, a no-op (the
//                          output task computes the down rows itself)
//   O_PROJ, MOE_COMBINE and the fused residual add + RMSNorm
//                       -> OP_OUT, one task per residual row tile: the tile's O-proj rows
//                          over every KV group, the experts' rows weighted by the router
//                          scores (its own down GEMV over every active expert at small
//                          batch, else the sum of the OP_MOE_DOWN partials), and h_{l+1}
//                          with the tile's sum of squares (consumers apply the norm)
//   LM_HEAD             -> OP_LM_HEAD; OP_EMBED seeds the residual stream.
enum Opcode : int32_t {
  OP_NOP = 0,
  OP_EMBED = 1,
  OP_QKV = 2,
  OP_ROUTER = 3,
  OP_ATTN = 4,
  OP_MOE_UP = 5,
  OP_OUT = 6,
  OP_LM_HEAD = 7,
  OP_MOE_DOWN = 8,
  OP_COUNT = 9,
};

// ---------------------------------------------------------------- descriptor
// 32 int32 per task, 128 bytes, read with scalar loads.  The pages' descriptor also
// carries the barrier to wait on, its target and the barrier to signal; here every data
// edge is a tagged word that the consumer polls, so those fields do not exist and words
// 8..31 are zero (reserved).
enum DescField : int32_t {
  D_OPCODE = 0,
  D_LAYER = 1,
  D_ARG0 = 2,   // first row / tile index / claimer index
  D_ARG1 = 3,   // row count / kv group / claimer count
  D_ARG2 = 4,
  D_ARG3 = 5,
  D_WAVE = 6,   // wave id in the schedule (for the op-per-kernel ablation)
  D_GIDX = 7,   // position in the global (flattened) order
  D_WORDS = 32,
};

// ---------------------------------------------------------------- counters
// Per-layer block of counters; all zeroed before each step.  Data edges travel as tagged
// words (no counter); the counters left are the heads of the two claim queues.
struct CounterLayout {
  int32_t per_layer;   // counters per layer block
  int32_t attn_claim;  // attention queue head
  int32_t up_claim;    // MoE up queue head
  int32_t down_claim;  // MoE down queue head
  int32_t global_base; // start of the step-global block (after n_layers+1 layer blocks)
  int32_t total;       // total counters
};

// Step-global status block (not per layer), at counters[global_base + ...].
enum GlobalCounter : int32_t {
  G_ABORT = 0,     // nonzero: a wait timed out; every workgroup stops
  G_ERR_CODE = 1,  // first error code (1 = watchdog, 2 = bad page-table entry)
  G_ERR_TASK = 2,  // global index of the task that reported it
  G_ERR_CTR = 3,   // counter index it waited on
  G_ERR_SEEN = 4,  // value observed
  G_ERR_WANT = 5,  // target
  G_DONE_WGS = 6,  // workgroups that finished their list
  G_TAGGED = -2,   // G_ERR_CTR value of a wait on tagged data (no counter)
  G_COUNT = 8,
};

// Words of one layer's published routing table (the LDS routing area's layout).
constexpr int32_t kRouteTableWords = 1548;
// Batch from which the expert down rows are computed by the MoE-down items (OP_MOE_DOWN)
// instead of inside the output tasks; a schedule built for smaller batches has no MoE-down
// tasks.
#ifndef MKD_DOWN_SPLIT_BATCH
#define MKD_DOWN_SPLIT_BATCH 2
#endif
constexpr int32_t kDownSplitBatch = MKD_DOWN_SPLIT_BATCH;

// ---------------------------------------------------------------- plan constants
struct PlanShape {
  int32_t n_rt;            // residual row tiles (hidden / rt_rows)
  int32_t rt_rows;         // rows per residual row tile
  int32_t up_rows;         // activation rows per MoE-up item (gate+up = 2x rows of weights)
  int32_t n_up_tiles;      // moe_inter / up_rows
  int32_t pages_per_item;  // attention pages per claimed item
  int32_t qkv_rows;        // weight rows per QKV tile (RoPE pairs kept together)
  int32_t qkv_tph;         // QKV tiles per head
  int32_t router_rows;     // rows per router tile
  int32_t lm_rows;         // rows per LM-head tile
  int32_t down_rows;       // expert down rows per OP_MOE_DOWN item
  int32_t n_down_chunks;   // hidden / down_rows
};

// ---------------------------------------------------------------- kernel parameters
struct Params {
  // geometry
  int32_t n_layers, hidden, n_q, n_kv, head_dim, n_experts, top_k, inter, vocab, page;
  float rms_eps;
  int32_t batch, max_batch, max_pages, n_pages;
  PlanShape shape;
  CounterLayout ctr;
  // weights (bf16)
  const uint16_t* embed;
  const uint16_t* norm;
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const uint16_t* w_router;
  const uint16_t* w_gate_up;
  const uint16_t* w_down;
  // per-step inputs
  const int32_t* tokens;
  const int32_t* seq_lens;
  const int32_t* page_table;
  uint16_t* kv_pool;
  float* logits;
  // workspace (fp32 unless noted)
  uint64_t* h;        // [L+1][maxB][H] tagged
  uint64_t* ss;       // [L+1][maxB][n_rt] tagged per-row-tile sums of squares
  uint64_t* q;        // [L][maxB][nq*hd] tagged post-RoPE queries
  uint64_t* kvflag;   // [L][2*nkv][64] tagged: K/V tile t of a head has stored its new slots
  uint64_t* attn_part;  // [max_items][hpg][hd + 2] tagged: unnormalised o, then m, l
  uint64_t* attn_o;     // [L][maxB][nq*hd] tagged
  uint64_t* router;   // [L][maxB][E] tagged
  uint64_t* route_tbl;  // [L][route words] tagged routing tables (built once per layer)
  int32_t* topk_ids;  // [L][maxB][k]
  float* topk_w;      // [L][maxB][k]
  uint64_t* moe_act;  // [L][maxB*k][I] tagged
  uint64_t* moe_part; // [maxB*k][H] tagged: an expert's output rows per (token, choice)
  const double* inv_freq;  // [hd/2] RoPE frequencies base^(-2i/hd), fp64
  uint64_t* rope;          // [maxB][hd/2][2] tagged cos, sin of this step's positions
  const void* dummy;       // 1 KB of zeros: target of the GEMV ring's idle slots
  uint32_t* counters;
  // task lists
  const int32_t* tasks;      // [n_tasks][32]
  const int32_t* cu_offsets; // [n_wg + 1]: task list of workgroup i
  int32_t max_attn_items;    // capacity of attn_part
  int32_t spin_limit;        // watchdog: polls before a wait gives up
  uint32_t epoch;            // this step's number in [1, 2^24): tagged words carry (epoch << 8) | layer
  // optional per-task trace: trace[gidx][4] = {start, inputs ready, end, meta}
  // (100 MHz wall clock; meta = opcode | workgroup << 8 | claimed items << 20 |
  //  (inputs staged - start) << 32 | (workers done - start) << 48, both in clock ticks)
  uint64_t* trace;
  int32_t trace_cap;         // tasks the trace buffer holds
  // local-attention layers: layer l attends to its last attn_window positions when
  // attn_window > 0 and (l + 1) % full_every != 0, to every position otherwise
  int32_t attn_window;
  int32_t full_every;
};

}  // namespace mkd
