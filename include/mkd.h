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
 * (Cohere).  Each call below names the section of that page it follows.
 *
 * Conventions
 *  - Every function returns MKD_OK (0) or a negative MKD_ERR_* code; the text of the
 *    last error of an engine is returned by mkd_last_error().  Nothing throws.
 *  - Device pointers are plain `void*` / typed pointers into the memory of the HIP
 *    device given to mkd_create(); streams are `hipStream_t` passed as `void*`
 *    (NULL = the default stream).
 *  - Ownership: the caller owns every device buffer: weights, KV pool, page tables,
 *    token ids, sequence lengths, logits, the trace buffer and the engine's workspace
 *    (sized by mkd_workspace_bytes, handed over with mkd_set_workspace).  The engine
 *    owns only host memory (its schedule and configuration) and never frees caller
 *    memory.  mkd_decode_step allocates nothing and makes no synchronous copy.
 *  - An engine is used from one host thread at a time.  Two engines must not share a
 *    workspace.
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

/* Model geometry (section "Where the speedup comes from": parallel layers whose
   attention and MoE read one normalised input; section "Tasks": 128 experts, top-k
   routing, SwiGLU experts; Figure 7: grouped-query attention with 4 KV groups).
   page_size is the number of tokens per paged-KV page. */
typedef struct mkd_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, moe_inter, vocab, page_size;
  float rms_eps, rope_base;
} mkd_config;

/* Device weights, bf16, row-major [out][in].  BORROWED: they must stay valid and
   unchanged while the engine uses them.
     embed     [vocab][hidden]                         token embedding, tied LM head
     norm      [n_layers+1][hidden]                    RMSNorm gains; gain_l feeds
                                                       layer l, gain_L the LM head
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

/* Create an engine for `cfg` on HIP device `hip_device`, able to decode batches of up
   to `max_batch` sequences whose page-table rows hold `max_pages_per_seq` entries
   (section "The serving engine around the kernel": the batch size and the page
   tables are the per-step inputs; section "The task scheduler: mapping tasks to SMs":
   the host builds the task lists once, here in mkd_create).  No device memory is
   allocated.  Geometry limits (the kernel is compiled for these row lengths):
   (hidden, moe_inter, head_dim) in {(2048, 768, 128), (256, 128, 64)},
   n_q_heads * head_dim a multiple (1 to 4) of hidden, n_q_heads / n_kv_heads <= 16,
   n_kv_heads <= 16, n_experts <= 256, top_k <= 16, page_size == 16, max_batch <= 16,
   max_pages_per_seq <= 24576.  hip_device = -1 creates a host-only engine (plan
   inspection, no decoding).  On error *out is set to NULL and MKD_ERR_ARG (bad
   configuration) or MKD_ERR_HIP is returned. */
int mkd_create(const mkd_config* cfg, int32_t hip_device, int32_t max_batch,
               int32_t max_pages_per_seq, mkd_engine** out);

/* Release the engine's host memory.  Caller memory (workspace included) is never
   freed.  NULL is ignored. */
void mkd_destroy(mkd_engine* eng);

/* Bytes of device workspace the engine needs: the tagged activation words of every
   layer, the attention partials, the claim counters, the RoPE frequencies and the
   task lists (section "Barriers": counters and per-step state in global memory;
   section "The task descriptor": the task lists the kernel reads).  Depends only on
   the configuration, max_batch and max_pages_per_seq.  0 for a host-only engine. */
size_t mkd_workspace_bytes(const mkd_engine* eng);

/* Hand the engine its workspace: `dev_ptr` is device memory of at least
   mkd_workspace_bytes() bytes, 256-byte aligned, owned by the caller and BORROWED
   until mkd_destroy or the next mkd_set_workspace.  The call clears it and copies the
   task lists and RoPE frequencies into it, then waits for those copies (a
   configuration call, not a per-step one; section "The serving engine around the
   kernel": per-step state is cleared on the device, the schedule is chosen by the
   host).  MKD_ERR_ARG for a NULL, misaligned or too small buffer. */
int mkd_set_workspace(mkd_engine* eng, void* dev_ptr, size_t bytes);

/* Record the weight pointers (no copy).  Returns MKD_ERR_ARG on a NULL pointer
   (section "Performance": bf16 weights streamed from HBM every step). */
int mkd_load_weights(mkd_engine* eng, const mkd_weights* w);

/* Choose MKD_MODE_MEGAKERNEL or MKD_MODE_OP_PER_KERNEL for later steps (section
   "Where the speedup comes from": the launch and synchronisation gaps between per-op
   kernels that the megakernel removes; the ablation runs the same tile bodies with one
   launch per wave of tasks, so those gaps come back).
   MKD_ERR_ARG for another value. */
int mkd_set_mode(mkd_engine* eng, int32_t mode);

/* One decode step for a ragged batch (section "The serving engine around the kernel":
   the host updates the KV positions and page tables, clears per-step state, selects
   the schedule and launches; sampling is the caller's).
     stream        HIP stream (void*), the step is asynchronous on it
     batch         number of sequences, 1 <= batch <= max_batch
     d_tokens      [batch] int32 device: the token id fed to each sequence
     d_seq_lens    [batch] int32 device: cached tokens of each sequence; the new
                   token sits at this 0-based position and attends to positions
                   0..seq_len inclusive
     h_seq_lens    [batch] int32 host mirror of d_seq_lens (validation and the
                   per-step choice of attention item size)
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
   Allocates nothing; the only host work is validation and two kernel launches (a
   counter clear and the step kernel).  Errors: MKD_ERR_STATE before
   mkd_load_weights or mkd_set_workspace, MKD_ERR_CAPACITY for batch > max_batch or a
   sequence longer than max_pages_per_seq pages, MKD_ERR_ARG for a bad argument
   (including a used page-table entry outside [0, n_pages) when h_page_table is given),
   MKD_ERR_HIP on a launch failure.  On the device, a page-table entry or token id out
   of range, or a sequence length past the page-table row, is never dereferenced; it is
   reported by mkd_sync_status(). */
int mkd_decode_step(mkd_engine* eng, void* stream, int32_t batch, const int32_t* d_tokens,
                    const int32_t* d_seq_lens, const int32_t* h_seq_lens,
                    const int32_t* d_page_table, const int32_t* h_page_table, void* kv_pool,
                    int32_t n_pages, float* d_logits);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc): the same step as mkd_decode_step,
   same arguments and errors, with the engine's workspace placed in a library-owned
   static device array of MKD_STATIC_SCRATCH_BYTES on each device instead of a caller
   buffer (mkd_set_workspace is not needed).  It calls no hipMalloc or hipFree.
   MKD_ERR_CAPACITY if mkd_workspace_bytes(eng) exceeds MKD_STATIC_SCRATCH_BYTES.  Every
   call on one GPU shares that GPU's array, which keeps the last call's contents until
   the process ends; a call from another engine than the last one to use the array
   clears it and copies its schedule in first (in order on `stream`).  Calls that overlap
   on one GPU (other streams or host threads) race: serialise them.  mkd_sync_status
   reports the errors of the last step of either kind; mkd_debug_read reads only the
   engine's own workspace. */
#define MKD_STATIC_SCRATCH_BYTES (64u << 20)
int mkd_decode_step_static(mkd_engine* eng, void* stream, int32_t batch, const int32_t* d_tokens,
                           const int32_t* d_seq_lens, const int32_t* h_seq_lens,
                           const int32_t* d_page_table, const int32_t* h_page_table, void* kv_pool,
                           int32_t n_pages, float* d_logits);

/* Wait for the engine's last step on its stream and report device-side errors
   (section "How do you write a megakernel?": a dependency that is counted wrong shows
   up as a wait that never ends, so every wait here has a bound):
   MKD_ERR_DEADLOCK if the wait watchdog fired (a dependency's data never arrived),
   MKD_ERR_ARG if an input was out of range on the device, else MKD_OK.  The error
   record is cleared.  Synchronous (a status call, not part of a step). */
int mkd_sync_status(mkd_engine* eng);

/* Watchdog bound of the kernel's waits: the number of polls after which a wait on data
   that never arrives gives up, marks the step failed (MKD_ERR_DEADLOCK from
   mkd_sync_status) and makes every workgroup leave the step (section "Barriers": a
   waiter spins until its dependency is met).  Default 4000000 (seconds of waiting);
   MKD_ERR_ARG unless 1 <= polls. */
int mkd_set_watchdog(mkd_engine* eng, int32_t polls);

/* Local-attention layers, the model variant of layers that are not full attention (the
   page's section "Tasks": the attention drain runs "only for full-attention layers").
   With window > 0, layer l attends to the last `window` positions of each sequence
   (positions pos - window + 1 .. pos, the new token's position pos included) unless
   (l + 1) % full_every == 0, in which case it attends to every position; window = 0
   (the default) makes every layer full attention.  The KV cache keeps every position.
   Applies to the following steps.  MKD_ERR_ARG unless window >= 0 and full_every >= 1. */
int mkd_set_attention_window(mkd_engine* eng, int32_t window, int32_t full_every);

/* Text of the engine's last error ("" if none).  The pointer stays valid until the
   next call on the engine.  With eng == NULL returns the last creation error. */
const char* mkd_last_error(const mkd_engine* eng);

/* Debug read-back of the last step's intermediate values (synchronous copy to the host
   buffer dst of `bytes` bytes; MKD_ERR_ARG if too small).  Section "Tasks" names the
   operations whose outputs these are:
     MKD_DEBUG_HIDDEN   fp32 [n_layers+1][batch][hidden]  residual entering each layer
                        and after the last one
     MKD_DEBUG_TOPK_IDS int32 [n_layers][batch][top_k]    selected experts, descending
     MKD_DEBUG_TOPK_W   fp32  [n_layers][batch][top_k]    their routing weights
     MKD_DEBUG_ROUTER   fp32  [n_layers][batch][n_experts] router logits
     MKD_DEBUG_Q        fp32  [n_layers][batch][nq*hd]    queries after RoPE (QKV_PROJ)
     MKD_DEBUG_ATTN     fp32  [n_layers][batch][nq*hd]    attention output per head,
                        after the merge of the page chunks (ATTN_DECODE + ATTN_COMBINE)
     MKD_DEBUG_ROUTE    int32 [n_layers][MKD_ROUTE_WORDS] routing table of each layer
                        (ROUTE_FINALIZE / MOE_GATHER), words:
                          [b*16 + j]          expert of choice j of token b
                          [256 + b*16 + j]    its routing weight (fp32 bits)
                          [512]               n_act, the number of distinct experts
                          [520 + a]           active expert a, ascending (a < n_act)
                          [776 + a]           start of expert a's entries (a <= n_act)
                          [1036 + i]          entry i = b*top_k + j, experts ascending,
                                              tokens ascending within an expert
                          [1292 + b*top_k + j] (active index << 16) | position of the
                                              entry in its expert's list
     MKD_DEBUG_ACT      fp32  [n_layers][batch*top_k][moe_inter] expert activation
                        silu(gate) * up of choice j of token b at row b*top_k + j
                        (MOE_UPGATE_ACT)                                                */
#define MKD_DEBUG_HIDDEN 0
#define MKD_DEBUG_TOPK_IDS 1
#define MKD_DEBUG_TOPK_W 2
#define MKD_DEBUG_ROUTER 3
#define MKD_DEBUG_Q 4
#define MKD_DEBUG_ATTN 5
#define MKD_DEBUG_ROUTE 6
#define MKD_DEBUG_ACT 7
#define MKD_ROUTE_WORDS 1548
int mkd_debug_read(mkd_engine* eng, int32_t what, void* dst, size_t bytes);

/* Optional per-task trace of later steps (section "How do you write a megakernel?",
   its last step: task order and placement are tuned for throughput, which needs the
   time line of every task on every CU).  dev_buf is a device buffer of
   `bytes` bytes receiving, for the task at global index i of the schedule, four uint64
   at offset 32*i: wall-clock (100 MHz) start, time its first wait on input data
   completed, end, and meta = opcode (8 bits) | CU << 8 (12 bits) | claimed items << 20
   (12 bits) | ticks from start until the inputs were staged << 32 (16 bits) | ticks
   from start until the compute finished << 48 (16 bits).  Tasks beyond the buffer are
   not recorded.  dev_buf = NULL disables it.  The caller owns the buffer. */
int mkd_set_trace(mkd_engine* eng, void* dev_buf, size_t bytes);

/* Message-passing litmus test of the step's inter-workgroup protocol on device
   hip_device (section "Barriers": producers publish, consumers spin until the dependency
   is met, and the fences must leave no data race across SMs; here across XCDs).
   n_pairs producer / consumer pairs of workgroups (2p, 2p + 1: on different XCDs) run
   `rounds` rounds over the same buffers, with the step's own primitives: 256 tagged
   words (agent-scope 64-bit stores and loads; the consumer checks the value of every word
   whose tag is the round) and 512 bf16 words published by agent-scope 16-bit stores, the
   producer's wait for them and a tagged flag, read after the flag and an agent-scope
   acquire with the non-temporal 16-byte loads that read K/V pages.  h_result[4]: words
   whose tag was new and value old, data words read stale after flag and acquire, waits
   that timed out, rounds the consumers completed.  Allocates and frees its buffers (a
   test call, not for a decode loop).  MKD_ERR_ARG unless 1 <= n_pairs <= 4096 and
   1 <= rounds <= 100000; MKD_ERR_HIP on a runtime error. */
int mkd_protocol_litmus(int32_t hip_device, int32_t n_pairs, int32_t rounds, uint32_t* h_result);

/* ---------------------------------------------------------------- continuous decode
   The loop around the step (section "The serving engine around the kernel": each step
   updates the KV positions and page tables, clears the step state, selects the schedule
   by the longest live context, launches, samples and retires finished sequences, while
   others join; a sequence that cannot get a KV page waits).  A server borrows an engine
   (which must outlive it and have its weights and workspace set) and manages n_pages
   physical pages of a caller-owned KV pool laid out as for mkd_decode_step.

   mkd_server_create     up to max_live (<= 4096) live sequences; allocates only pinned
                         host staging (two copies of the step's upload) at creation.  Over
                         a host-only engine the server does every step's scheduling and
                         bookkeeping without launching (kv_pool may be NULL, no buffer;
                         mkd_server_last_step reports fed = the first token of a new
                         sequence, else -1, and sampled = -1).
   mkd_server_buffer_bytes / mkd_server_set_buffer
                         a caller-owned device buffer (256-byte aligned) for the step's
                         inputs, the logits [max_batch][vocab] fp32 and the sampled tokens;
                         settable while no sequence is live.
   mkd_server_join       a sequence with cached_len tokens already in the cache, fed
                         first_token at position cached_len, generating max_new_tokens
                         tokens (greedy); ceil(cached_len / page_size) pages are taken
                         from the free list now and written to h_pages (the caller fills
                         them with the cached K/V, ordered after the previous step on
                         its stream).  MKD_ERR_CAPACITY when max_live sequences are live
                         or too few pages are free (nothing is taken), MKD_ERR_ARG for a
                         duplicate id or a sequence longer than max_pages_per_seq pages.
   mkd_server_step       one step on `stream`: the live sequences in join order, up to
                         the engine's max_batch; a sequence whose next token opens a page
                         takes a free page or is parked (keeps its pages, skipped) until
                         one is free.  Feeds each sequence its first token or its last
                         sampled token, runs mkd_decode_step, samples every row with an
                         argmax (ties to the lower id), retires the sequences that have
                         generated their tokens (their pages return to the free list).
                         Asynchronous: one upload and one download on the stream, no
                         allocation.  *n_scheduled = the step's batch (0 when nothing is
                         live).  MKD_ERR_CAPACITY when every live sequence is parked;
                         errors of mkd_decode_step are passed on.
   mkd_server_last_step  waits for the last step and reports its batch: sequence ids,
                         tokens fed, tokens sampled, seq_lens (the fed token's position),
                         page-table rows [batch][max_pages_per_seq] and, when logits is
                         not NULL, the logits [batch][vocab] (a synchronous copy); any
                         output pointer may be NULL.
   mkd_server_stats      live and parked sequences, free pages. */
typedef struct mkd_server mkd_server;
int mkd_server_create(mkd_engine* eng, int32_t n_pages, int32_t max_live, mkd_server** out);
void mkd_server_destroy(mkd_server* srv);
size_t mkd_server_buffer_bytes(const mkd_server* srv);
int mkd_server_set_buffer(mkd_server* srv, void* dev_ptr, size_t bytes);
int mkd_server_join(mkd_server* srv, int64_t seq_id, int32_t cached_len, int32_t first_token,
                    int32_t max_new_tokens, int32_t* h_pages, int32_t max_pages_out);
int mkd_server_step(mkd_server* srv, void* stream, void* kv_pool, int32_t* n_scheduled);
int mkd_server_last_step(mkd_server* srv, int64_t* ids, int32_t* fed, int32_t* sampled, int32_t* seq_lens,
                         int32_t* page_table, float* logits, int32_t max_batch_out, int32_t* batch);
int mkd_server_stats(const mkd_server* srv, int32_t* n_live, int32_t* n_parked, int32_t* n_free_pages);
const char* mkd_server_last_error(const mkd_server* srv);

/* Schedule of the engine's task lists (section "The task scheduler: mapping tasks to
   SMs": the wave order and the placement of tasks on SMs; every schedule that keeps each
   producer wave ahead of its consumers computes the same step, bit for bit, because every
   task waits only on tasks earlier in the global order and every reduction has a fixed
   order).  order: MKD_ORDER_*; placement: MKD_PLACE_* (workgroup w runs on XCD w mod 8;
   XCD placement puts runs of n_cu / 8 consecutive tasks on one XCD).  Rebuilds the lists
   and, when a workspace is set, uploads them synchronously (a set-up call, not for the
   decode loop; the next step starts a new epoch).  Also applies to mkd_plan_inspect.
   MKD_ERR_ARG for an unknown order or placement, or an XCD placement on a device whose
   compute-unit count is not a multiple of 8. */
#define MKD_ORDER_DEFAULT 0     /* qkv, router, attention, MoE-up, output */
#define MKD_ORDER_ATTN_FIRST 1  /* qkv, attention, router, MoE-up, output */
#define MKD_ORDER_MOE_FIRST 2   /* router, qkv, MoE-up, attention, output */
#define MKD_ORDER_INTERLEAVED 3 /* qkv, router, attention and MoE-up claimers alternating, output */
#define MKD_PLACE_ROUND_ROBIN 0
#define MKD_PLACE_XCD 1
int mkd_set_schedule(mkd_engine* eng, int32_t order, int32_t placement);

/* Plan inspection (host only; works on an engine created with hip_device = -1): writes
   the task descriptors the scheduler builds onto `n_cu` compute units (section "The
   task scheduler: mapping tasks to SMs"; section "The task descriptor": 32 int32 per
   task, field 0 the opcode).  desc receives n_tasks * 32 int32, list after list, each
   in execution order; cu_offsets (room for n_cu + 1 entries) receives the start of
   each CU's list and the total.  *n_tasks is set to the total; MKD_ERR_CAPACITY if
   max_tasks is too small.  The schedule does not depend on the batch size.  The
   descriptor fields are documented in decode_megakernel_amd/csrc/mkd_common.h. */
int mkd_plan_inspect(mkd_engine* eng, int32_t n_cu, int32_t* desc, int32_t max_tasks,
                     int32_t* cu_offsets, int32_t* n_tasks);

#ifdef __cplusplus
}
#endif

#endif /* MKD_H */
