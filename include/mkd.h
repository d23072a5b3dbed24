/*
 * mkd.h - C-ABI of the persistent decode megakernel for AMD Instinct MI355X (gfx950).
 *
 * One call runs one whole autoregressive decode step of a parallel-transformer MoE
 * model as a single persistent kernel: one workgroup per compute unit, resident for
 * the step, walking a host-built per-CU task list (one task = one tile of one op),
 * with dependencies carried through global memory (tagged 64-bit data words whose
 * tag names the step and layer, polled by their consumers; atomic counters for the
 * shared claim queues) and the variable-size attention and MoE work balanced over
 * the compute units.
 *
 * Source of the method: "Inside the megakernel serving engine for North Mini Code"
 * (Cohere), sections "What is a Megakernel?" (persistent kernel, per-SM task lists,
 * counters in global memory), "Tasks" and "The task descriptor" (opcodes, 32-int32
 * descriptors), "Barriers" (wait = spin until count >= target, arrive = fence then
 * atomic add), "The task scheduler: mapping tasks to SMs" (named waves dealt round
 * robin, claimers on shared queues), "The serving engine around the kernel" (the
 * host loop updates KV positions, clears per-step state, selects a schedule,
 * launches, samples), and "Performance" (batch-1 decode against a synthetic KV
 * cache).
 *
 * Conventions
 *  - Every function returns MKD_OK (0) or a negative MKD_ERR_* code; the text of the
 *    last error of an engine is returned by mkd_last_error().  Nothing throws.
 *  - Device pointers are plain `void*` / typed pointers into the memory of the HIP
 *    device given to mkd_create(); streams are `hipStream_t` passed as `void*`
 *    (NULL = the default stream).
 *  - The caller owns every buffer it passes (weights, KV pool, page tables, token
 *    ids, sequence lengths, logits).  The engine owns only its own workspace
 *    (activations, counters, task lists) and frees it in mkd_destroy().
 *  - An engine is used from one host thread at a time.
 */
#ifndef MKD_H
#define MKD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MKD_OK 0
#define MKD_ERR_ARG (-1)       /* invalid argument (shape, pointer, capacity)            */
#define MKD_ERR_HIP (-2)       /* a HIP runtime call failed                               */
#define MKD_ERR_CAPACITY (-3)  /* request exceeds what the engine was created for        */
#define MKD_ERR_DEADLOCK (-4)  /* the device watchdog stopped a wait that never completed */
#define MKD_ERR_STATE (-5)     /* call out of order (e.g. decode before weights)         */

/* Execution modes of mkd_decode_step. */
#define MKD_MODE_MEGAKERNEL 0    /* one persistent cooperative launch per step (default) */
#define MKD_MODE_OP_PER_KERNEL 1 /* ablation: each wave of tasks is its own launch      */

/* Model geometry ("Where the speedup comes from": parallel layers; "Tasks": 128
   experts, top-k routing; Figure 7: 4 KV groups).  page_size is the number of
   tokens per paged-KV page. */
typedef struct mkd_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, moe_inter, vocab, page_size;
  float rms_eps, rope_base;
} mkd_config;

/* Device weights, bf16, row-major [out][in].  BORROWED: they must stay valid and
   unchanged while the engine uses them.
     embed     [vocab][hidden]                         token embedding, tied LM head
     norm      [n_layers+1][hidden]                    RMSNorm gammas; gamma_l feeds
                                                       layer l, gamma_L the LM head
     w_qkv     [n_layers][(nq+2*nkv)*hd][hidden]       rows: q heads | k heads | v heads
     w_o       [n_layers][hidden][nq*hd]
     w_router  [n_layers][n_experts][hidden]
     w_gate_up [n_layers][n_experts][2*inter][hidden]  rows: gate | up
     w_down    [n_layers][n_experts][hidden][inter]                                  */
typedef struct mkd_weights {
  const void* embed;
  const void* norm;
  const void* w_qkv;
  const void* w_o;
  const void* w_router;
  const void* w_gate_up;
  const void* w_down;
} mkd_weights;

typedef struct mkd_engine mkd_engine;

/* Create an engine for `cfg` on HIP device `hip_device`, able to decode batches of
   up to `max_batch` sequences whose page-table rows hold `max_pages_per_seq`
   entries.  Allocates the engine's device workspace.  Geometry limits (the kernel is
   compiled for these row lengths): hidden in {256, 2048}, n_q_heads * head_dim /
   n_kv_heads in {256, 1024}, moe_inter in {128, 768}, head_dim in {64, 128},
   n_q_heads / n_kv_heads <= 16, n_kv_heads <= 16, n_experts <= 256, top_k <= 16,
   page_size == 16, max_batch <= 16, max_pages_per_seq <= 24576.
   hip_device = -1 creates a host-only engine (plan inspection, no decoding).
   On error *out is set to NULL. */
int mkd_create(const mkd_config* cfg, int32_t hip_device, int32_t max_batch,
               int32_t max_pages_per_seq, mkd_engine** out);

/* Release the engine and its workspace (never caller memory).  NULL is ignored. */
void mkd_destroy(mkd_engine* eng);

/* Record the weight pointers (no copy).  Returns MKD_ERR_ARG on a NULL pointer. */
int mkd_load_weights(mkd_engine* eng, const mkd_weights* w);

/* Choose MKD_MODE_MEGAKERNEL or MKD_MODE_OP_PER_KERNEL for later steps. */
int mkd_set_mode(mkd_engine* eng, int32_t mode);

/* One decode step for a ragged batch ("The serving engine around the kernel").
     stream        HIP stream (void*), the step is asynchronous on it
     batch         number of sequences, 1 <= batch <= max_batch
     d_tokens      [batch] int32 device: the token id fed to each sequence
     d_seq_lens    [batch] int32 device: cached tokens of each sequence; the new
                   token sits at this 0-based position and attends to positions
                   0..seq_len inclusive
     h_seq_lens    [batch] int32 host mirror of d_seq_lens (validation and the
                   per-step schedule choice)
     d_page_table  [batch][max_pages_per_seq] int32 device: physical page of each
                   logical page; entries 0..seq_len/page_size must be valid pages
     h_page_table  optional host mirror of d_page_table (NULL to skip the host check
                   of every used entry against n_pages)
     kv_pool       device KV cache, bf16, [n_layers][2][n_pages][nkv][page*hd]; K pages
                   are token-major ([page][hd]), V pages dim-major ([hd][page]).  The
                   step writes the new token's k (after RoPE) and v into slot
                   (page_table[b][seq_len/page], seq_len % page) of every layer and
                   changes no other byte.
     n_pages       physical pages in kv_pool
     d_logits      [batch][vocab] fp32 device, written
   Errors: MKD_ERR_ARG for a bad argument (including a used page-table entry outside
   [0, n_pages) when h_page_table is given), MKD_ERR_STATE before mkd_load_weights,
   MKD_ERR_HIP on a launch failure.  A page-table entry found invalid on the device
   is skipped (never dereferenced) and reported by mkd_sync_status(). */
int mkd_decode_step(mkd_engine* eng, void* stream, int32_t batch, const int32_t* d_tokens,
                    const int32_t* d_seq_lens, const int32_t* h_seq_lens,
                    const int32_t* d_page_table, const int32_t* h_page_table, void* kv_pool,
                    int32_t n_pages, float* d_logits);

/* Wait for the engine's last step on its stream and report device-side errors:
   MKD_ERR_DEADLOCK if the wait watchdog fired (a dependency's data or counter
   never arrived), MKD_ERR_ARG if a page-table entry was out of range, else MKD_OK.
   The error record is cleared. */
int mkd_sync_status(mkd_engine* eng);

/* Text of the engine's last error ("" if none).  The pointer stays valid until the
   next call on the engine.  With eng == NULL returns the last creation error. */
const char* mkd_last_error(const mkd_engine* eng);

/* Debug read-back of the last step's intermediate values (synchronous copy to the
   host buffer dst of `bytes` bytes; MKD_ERR_ARG if too small):
     MKD_DEBUG_HIDDEN   fp32 [n_layers+1][batch][hidden]  residual entering each layer
                        and after the last one
     MKD_DEBUG_TOPK_IDS int32 [n_layers][batch][top_k]    selected experts, descending
     MKD_DEBUG_TOPK_W   fp32  [n_layers][batch][top_k]    their routing weights
     MKD_DEBUG_ROUTER   fp32  [n_layers][batch][n_experts] router logits        */
#define MKD_DEBUG_HIDDEN 0
#define MKD_DEBUG_TOPK_IDS 1
#define MKD_DEBUG_TOPK_W 2
#define MKD_DEBUG_ROUTER 3
int mkd_debug_read(mkd_engine* eng, int32_t what, void* dst, size_t bytes);

/* Optional per-task trace of later steps (the tracing subsystem): dev_buf is a device
   buffer of `bytes` bytes receiving, for the task at global index i of the step's
   schedule, four uint64 at offset 32*i: wall-clock (100 MHz) start, time its input
   counter was satisfied, end, and meta = opcode (8 bits) | task list << 8 (12 bits) |
   claimed items << 20 (12 bits) | ticks from start until the inputs were staged << 32
   (16 bits) | ticks from start until the compute finished << 48 (16 bits).  Tasks
   beyond the buffer are not recorded.  dev_buf = NULL disables it.
   The caller owns the buffer. */
int mkd_set_trace(mkd_engine* eng, void* dev_buf, size_t bytes);

/* Plan inspection (host only; works on an engine created with hip_device = -1):
   writes the task descriptors the scheduler builds for `batch` sequences onto
   `n_cu` compute units.  Each CU runs n_teams task lists side by side (1 or 2;
   *n_teams receives it if n_teams is not NULL); list cu * n_teams + t belongs to team
   t of CU cu.  desc receives n_tasks * 32 int32, list after list, each in execution
   order; cu_offsets (room for 2 * n_cu + 1 entries) receives the start of each list
   and the total.  *n_tasks is set to the total; MKD_ERR_CAPACITY if max_tasks is too
   small.  The descriptor layout (32 int32; field 0 = opcode) is documented in
   decode_megakernel_amd/csrc/mkd_common.h. */
int mkd_plan_inspect(mkd_engine* eng, int32_t batch, int32_t n_cu, int32_t* desc,
                     int32_t max_tasks, int32_t* cu_offsets, int32_t* n_tasks, int32_t* n_teams);

#ifdef __cplusplus
}
#endif

#endif /* MKD_H */
