/*
 * oracle.h - plain CPU reference of one decode step of the parallel-transformer
 * MoE model that the decode megakernel runs.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the GPU path.
 *
 * Source: "Inside the megakernel serving engine for North Mini Code" (Cohere),
 * sections "Where the speedup comes from" (parallel transformer layers: attention
 * and the MoE feed-forward read the same normalised input and are rejoined only by
 * a fused residual add + RMSNorm), "Tasks" (the opcode list: QKV with RoPE in the
 * epilogue, split-K decode attention plus combine, router scoring 128 experts,
 * per-token top-k, SiLU-and-multiply expert gate/up, expert down, MOE_COMBINE as
 * the router-score-weighted sum of a token's expert outputs, LM head) and Figure 7
 * (grouped-query attention with 4 KV groups).
 *
 * Precision: activations and accumulation in fp32, weights and the KV cache in
 * bf16 (widened exactly to fp32), RoPE angles in fp64.  Every loop runs in the
 * plain order of its definition; OpenMP only splits independent output rows.
 *
 * Layouts (shared contract with the library; documented in include/mkd.h):
 *   embed     [vocab][hidden]                         bf16, tied with the LM head
 *   norm      [n_layers+1][hidden]                    bf16 (gamma_0 .. gamma_L)
 *   w_qkv     [n_layers][(nq+2*nkv)*hd][hidden]       rows: q heads | k heads | v heads
 *   w_o       [n_layers][hidden][nq*hd]
 *   w_router  [n_layers][n_experts][hidden]
 *   w_gate_up [n_layers][n_experts][2*inter][hidden]  rows: gate | up
 *   w_down    [n_layers][n_experts][hidden][inter]
 *   kv pool   [n_layers][2][n_pages][nkv][page*hd]    bf16; K pages token-major
 *             ([page][hd]), V pages dim-major ([hd][page])
 */
#ifndef MKD_ORACLE_H
#define MKD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* attn_window / full_every: local-attention layers (the page's section "Tasks": the
   attention drain serves "only full-attention layers", so some layers are not).  In a
   decode step, layer l attends to the last attn_window positions when attn_window > 0
   and (full_every < 1 or (l + 1) % full_every != 0), to every position otherwise.
   orc_attention and orc_layer apply attn_window as given (0: every position). */
typedef struct orc_dims {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, moe_inter, vocab, page_size;
  float rms_eps, rope_base;
  int32_t attn_window, full_every;
} orc_dims;

float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);

/* out = v / sqrt(mean(v^2) + eps) * gamma. */
void orc_rmsnorm(int32_t n, const float* v, const uint16_t* gamma, float eps, float* out);

/* y[r] = sum_c W[r][c] * x[c], W bf16 row-major [rows][cols]. */
void orc_matvec_bf16(int32_t rows, int32_t cols, const uint16_t* W, const float* x, float* y);

/* Rotate-half RoPE of one head vector at position pos, in place. */
void orc_rope(int32_t head_dim, float base, int64_t pos, float* v);

/* Element index in the layer's pool slice of K (kv=0) or V (kv=1) for
   (physical page, kv group, token in page, dim). */
int64_t orc_kv_index(const orc_dims* d, int32_t n_pages, int32_t kv, int32_t page, int32_t g,
                     int32_t t, int32_t dim);

/* QKV projection, RoPE on q and k at position pos, and the bf16 write of the new
   k and v into the slot (page_row[pos / page], pos % page) of the layer's pool. */
void orc_qkv_rope_append(const orc_dims* d, int64_t pos, const int32_t* page_row, const float* x,
                         const uint16_t* w_qkv, uint16_t* kv_layer, int32_t n_pages, float* q);

/* Decode attention of every q head over positions 0..pos read through the page
   table, or over the last d->attn_window of them when attn_window > 0.  o is [nq][hd]. */
void orc_attention(const orc_dims* d, int64_t pos, const int32_t* page_row,
                   const uint16_t* kv_layer, int32_t n_pages, const float* q, float* o);

/* Top-k of n logits (descending, ties to the lower index) and the softmax of the
   selected logits. */
void orc_topk_softmax(int32_t n, int32_t k, const float* logits, int32_t* ids, float* w);

/* act = silu(W_gate x) * (W_up x) for one expert ("Tasks": MOE_UPGATE_ACT); w_gate_up is
   [2*inter][hidden], the gate rows first. */
void orc_expert_act(int32_t hidden, int32_t inter, const float* x, const uint16_t* w_gate_up, float* act);

/* y = W_down (silu(W_gate x) * (W_up x)) for one expert; w_gate_up is [2*inter][hidden]. */
void orc_expert_ffn(int32_t hidden, int32_t inter, const float* x, const uint16_t* w_gate_up,
                    const uint16_t* w_down, float* y);

/* m = sum_j w[j] * expert_ffn(ids[j])(x); expert e's weights at gate_up[e], down[e]. */
void orc_moe(const orc_dims* d, const float* x, const int32_t* ids, const float* w,
             const uint16_t* const* gate_up, const uint16_t* const* down, float* m);

/* One parallel-transformer layer for a batch; h [B][H] is updated in place.
   Optional outputs (NULL to skip): x_out [B][H] normed input, q_out [B][nq][hd],
   attn_out [B][nq*hd], router_out [B][E], ids_out/w_out [B][k]. */
void orc_layer(const orc_dims* d, int32_t batch, const int32_t* seq_lens,
               const int32_t* page_table, int32_t max_pages, uint16_t* kv_layer,
               int32_t n_pages, const uint16_t* gamma, const uint16_t* w_qkv,
               const uint16_t* w_o, const uint16_t* w_router, const uint16_t* w_gate_up,
               const uint16_t* w_down, float* h, float* x_out, float* q_out, float* attn_out,
               float* router_out, int32_t* ids_out, float* w_out);

/* One decode step: embedding, n_layers layers, final norm and tied LM head.
   logits [B][vocab].  h_layers (optional, [n_layers+1][B][H]) receives the
   residual stream entering each layer and after the last; ids_layers /
   w_layers (optional, [n_layers][B][k]) the routing. */
void orc_decode_step(const orc_dims* d, int32_t batch, const int32_t* tokens,
                     const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                     uint16_t* kv_pool, int32_t n_pages, const uint16_t* embed,
                     const uint16_t* norm, const uint16_t* w_qkv, const uint16_t* w_o,
                     const uint16_t* w_router, const uint16_t* w_gate_up,
                     const uint16_t* w_down, float* logits, float* h_layers,
                     int32_t* ids_layers, float* w_layers);

/* Final norm and LM head for a batch: logits[b] = embed . rmsnorm(h[b]; gamma). */
void orc_lm_head(const orc_dims* d, int32_t batch, const float* h, const uint16_t* gamma,
                 const uint16_t* embed, float* logits);

#ifdef __cplusplus
}
#endif

#endif /* MKD_ORACLE_H */
