/*
 * oracle.c - plain CPU reference of one decode step (see oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the decode library.
 *
 * Every function is the textbook definition of its step, written out with
 * plain loops in the order of that definition.  Passages cited are from the
 * page "Inside the megakernel serving engine for North Mini Code".
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

float orc_bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = ((uint32_t)b) << 16;
  return v.f;
}

uint16_t orc_f32_to_bf16(float f) {
  /* round to nearest, ties to even (the cache dtype is bf16). */
  union { float f; uint32_t u; } v;
  v.f = f;
  if ((v.u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((v.u >> 16) | ((v.u & 0xFFFFu) ? 0x40u : 0u));
  uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

/* RMSNorm, the normalisation that both branches share ("Where the speedup comes
   from": parallel layers rejoined by a fused residual add + RMSNorm). */
void orc_rmsnorm(int32_t n, const float* v, const uint16_t* gamma, float eps, float* out) {
  float ss = 0.0f;
  for (int32_t i = 0; i < n; ++i) ss += v[i] * v[i];
  const float inv = 1.0f / sqrtf(ss / (float)n + eps);
  for (int32_t i = 0; i < n; ++i) out[i] = v[i] * inv * orc_bf16_to_f32(gamma[i]);
}

/* Matrix-vector product with bf16 weights ("Tasks": every GEMM opcode computes
   output tiles of Y = X W). */
void orc_matvec_bf16(int32_t rows, int32_t cols, const uint16_t* W, const float* x, float* y) {
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < rows; ++r) {
    const uint16_t* w = W + (int64_t)r * cols;
    float acc = 0.0f;
    for (int32_t c = 0; c < cols; ++c) acc += orc_bf16_to_f32(w[c]) * x[c];
    y[r] = acc;
  }
}

/* Rotate-half RoPE ("Tasks": QKV_PROJ applies RoPE in its epilogue).  Pairs
   (i, i + hd/2) rotate by pos * base^(-2i/hd); angles are formed in fp64. */
void orc_rope(int32_t head_dim, float base, int64_t pos, float* v) {
  const int32_t half = head_dim / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double theta = pow((double)base, -2.0 * (double)i / (double)head_dim);
    const double ang = (double)pos * theta;
    const float c = (float)cos(ang);
    const float s = (float)sin(ang);
    const float a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

int64_t orc_kv_index(const orc_dims* d, int32_t n_pages, int32_t kv, int32_t page, int32_t g,
                     int32_t t, int32_t dim) {
  const int64_t P = d->page_size, D = d->head_dim;
  const int64_t base = (((int64_t)kv * n_pages + page) * d->n_kv_heads + g) * (P * D);
  return kv == 0 ? base + (int64_t)t * D + dim : base + (int64_t)dim * P + t;
}

/* QKV_PROJ ("Tasks"): [q; k; v] = W_qkv x, RoPE on q and k at the new token's
   position, and the new k, v stored (as bf16) into the token's paged-KV slot. */
void orc_qkv_rope_append(const orc_dims* d, int64_t pos, const int32_t* page_row, const float* x,
                         const uint16_t* w_qkv, uint16_t* kv_layer, int32_t n_pages, float* q) {
  const int32_t nq = d->n_q_heads, nkv = d->n_kv_heads, hd = d->head_dim, H = d->hidden;
  const int32_t rows = (nq + 2 * nkv) * hd;
  float* y = (float*)malloc(sizeof(float) * (size_t)rows);
  orc_matvec_bf16(rows, H, w_qkv, x, y);
  float* k = y + nq * hd;
  float* v = y + (nq + nkv) * hd;
  for (int32_t j = 0; j < nq; ++j) orc_rope(hd, d->rope_base, pos, y + j * hd);
  for (int32_t g = 0; g < nkv; ++g) orc_rope(hd, d->rope_base, pos, k + g * hd);
  memcpy(q, y, sizeof(float) * (size_t)nq * hd);
  const int32_t page = page_row[pos / d->page_size];
  const int32_t t = (int32_t)(pos % d->page_size);
  for (int32_t g = 0; g < nkv; ++g)
    for (int32_t e = 0; e < hd; ++e) {
      kv_layer[orc_kv_index(d, n_pages, 0, page, g, t, e)] = orc_f32_to_bf16(k[g * hd + e]);
      kv_layer[orc_kv_index(d, n_pages, 1, page, g, t, e)] = orc_f32_to_bf16(v[g * hd + e]);
    }
  free(y);
}

/* Decode attention ("Tasks": ATTN_DECODE over KV slices + ATTN_COMBINE is, by
   definition, plain softmax attention over the whole sequence; Figure 7: q head j
   reads KV group j / (nq / nkv)).  s_t = q . k_t / sqrt(hd), P = softmax(s),
   o = sum_t P_t v_t, positions 0..pos (the new token included); on a local-attention
   layer, positions pos - W + 1 .. pos only (W = d->attn_window > 0). */
void orc_attention(const orc_dims* d, int64_t pos, const int32_t* page_row,
                   const uint16_t* kv_layer, int32_t n_pages, const float* q, float* o) {
  const int32_t nq = d->n_q_heads, hd = d->head_dim, P = d->page_size;
  const int32_t group = nq / d->n_kv_heads;
  const int64_t t0 = (d->attn_window > 0 && pos + 1 > d->attn_window) ? pos + 1 - d->attn_window : 0;
  const int64_t n = pos + 1 - t0;  /* positions t0 .. pos; s[i] belongs to position t0 + i */
  const float scale = 1.0f / sqrtf((float)hd);
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < nq; ++j) {
    const int32_t g = j / group;
    const float* qj = q + (int64_t)j * hd;
    float* s = (float*)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
      const int64_t t = t0 + i;
      const int32_t page = page_row[t / P], tt = (int32_t)(t % P);
      float dot = 0.0f;
      for (int32_t e = 0; e < hd; ++e)
        dot += qj[e] * orc_bf16_to_f32(kv_layer[orc_kv_index(d, n_pages, 0, page, g, tt, e)]);
      s[i] = dot * scale;
    }
    float mx = s[0];
    for (int64_t t = 1; t < n; ++t) mx = s[t] > mx ? s[t] : mx;
    float sum = 0.0f;
    for (int64_t t = 0; t < n; ++t) {
      s[t] = expf(s[t] - mx);
      sum += s[t];
    }
    for (int64_t t = 0; t < n; ++t) s[t] /= sum;
    float* oj = o + (int64_t)j * hd;
    for (int32_t e = 0; e < hd; ++e) oj[e] = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t t = t0 + i;
      const int32_t page = page_row[t / P], tt = (int32_t)(t % P);
      for (int32_t e = 0; e < hd; ++e)
        oj[e] += s[i] * orc_bf16_to_f32(kv_layer[orc_kv_index(d, n_pages, 1, page, g, tt, e)]);
    }
    free(s);
  }
}

/* ROUTER_TOPK ("Tasks": top-k experts per token).  Selection by descending logit,
   ties to the lower expert index; the weights are the softmax of the selected
   logits (equal to the full softmax renormalised over the selection). */
void orc_topk_softmax(int32_t n, int32_t k, const float* logits, int32_t* ids, float* w) {
  char* taken = (char*)calloc((size_t)n, 1);
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < n; ++e)
      if (!taken[e] && (best < 0 || logits[e] > logits[best])) best = e;
    taken[best] = 1;
    ids[j] = best;
  }
  free(taken);
  const float mx = logits[ids[0]];
  float sum = 0.0f;
  for (int32_t j = 0; j < k; ++j) {
    w[j] = expf(logits[ids[j]] - mx);
    sum += w[j];
  }
  for (int32_t j = 0; j < k; ++j) w[j] /= sum;
}

/* One expert ("Tasks": MOE_UPGATE_ACT fuses SiLU-and-multiply into the gate/up
   GEMM, MOE_DOWN projects back). */
void orc_expert_act(int32_t hidden, int32_t inter, const float* x, const uint16_t* w_gate_up, float* act) {
  float* gu = (float*)malloc(sizeof(float) * 2 * (size_t)inter);
  orc_matvec_bf16(2 * inter, hidden, w_gate_up, x, gu);
  for (int32_t i = 0; i < inter; ++i) {
    const float g = gu[i];
    const float silu = g / (1.0f + expf(-g));
    gu[i] = silu * gu[inter + i];
  }
  memcpy(act, gu, sizeof(float) * (size_t)inter);
  free(gu);
}

void orc_expert_ffn(int32_t hidden, int32_t inter, const float* x, const uint16_t* w_gate_up,
                    const uint16_t* w_down, float* y) {
  float* act = (float*)malloc(sizeof(float) * (size_t)inter);
  orc_expert_act(hidden, inter, x, w_gate_up, act);
  orc_matvec_bf16(hidden, inter, w_down, act, y);
  free(act);
}

/* MoE feed-forward ("Tasks": MOE_COMBINE sums a token's expert outputs weighted
   by the router scores). */
void orc_moe(const orc_dims* d, const float* x, const int32_t* ids, const float* w,
             const uint16_t* const* gate_up, const uint16_t* const* down, float* m) {
  const int32_t H = d->hidden;
  float* y = (float*)malloc(sizeof(float) * (size_t)H);
  for (int32_t i = 0; i < H; ++i) m[i] = 0.0f;
  for (int32_t j = 0; j < d->top_k; ++j) {
    orc_expert_ffn(H, d->moe_inter, x, gate_up[ids[j]], down[ids[j]], y);
    for (int32_t i = 0; i < H; ++i) m[i] += w[j] * y[i];
  }
  free(y);
}

/* One parallel-transformer layer ("Where the speedup comes from": attention and
   the MoE read the same normalised input; their outputs rejoin the residual). */
void orc_layer(const orc_dims* d, int32_t batch, const int32_t* seq_lens,
               const int32_t* page_table, int32_t max_pages, uint16_t* kv_layer,
               int32_t n_pages, const uint16_t* gamma, const uint16_t* w_qkv,
               const uint16_t* w_o, const uint16_t* w_router, const uint16_t* w_gate_up,
               const uint16_t* w_down, float* h, float* x_out, float* q_out, float* attn_out,
               float* router_out, int32_t* ids_out, float* w_out) {
  const int32_t H = d->hidden, nq = d->n_q_heads, hd = d->head_dim, E = d->n_experts;
  const int32_t K = d->top_k, I = d->moe_inter;
  float* x = (float*)malloc(sizeof(float) * (size_t)H);
  float* q = (float*)malloc(sizeof(float) * (size_t)nq * hd);
  float* o = (float*)malloc(sizeof(float) * (size_t)nq * hd);
  float* a = (float*)malloc(sizeof(float) * (size_t)H);
  float* r = (float*)malloc(sizeof(float) * (size_t)E);
  float* m = (float*)malloc(sizeof(float) * (size_t)H);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  float* w = (float*)malloc(sizeof(float) * (size_t)K);
  const uint16_t** gu = (const uint16_t**)malloc(sizeof(void*) * (size_t)E);
  const uint16_t** dn = (const uint16_t**)malloc(sizeof(void*) * (size_t)E);
  for (int32_t e = 0; e < E; ++e) {
    gu[e] = w_gate_up + (int64_t)e * 2 * I * H;
    dn[e] = w_down + (int64_t)e * H * I;
  }
  for (int32_t b = 0; b < batch; ++b) {
    float* hb = h + (int64_t)b * H;
    const int64_t pos = seq_lens[b];
    const int32_t* row = page_table + (int64_t)b * max_pages;
    orc_rmsnorm(H, hb, gamma, d->rms_eps, x);
    orc_qkv_rope_append(d, pos, row, x, w_qkv, kv_layer, n_pages, q);
    orc_attention(d, pos, row, kv_layer, n_pages, q, o);
    orc_matvec_bf16(H, nq * hd, w_o, o, a);
    orc_matvec_bf16(E, H, w_router, x, r);
    orc_topk_softmax(E, K, r, ids, w);
    orc_moe(d, x, ids, w, gu, dn, m);
    for (int32_t i = 0; i < H; ++i) hb[i] = hb[i] + a[i] + m[i];
    if (x_out) memcpy(x_out + (int64_t)b * H, x, sizeof(float) * (size_t)H);
    if (q_out) memcpy(q_out + (int64_t)b * nq * hd, q, sizeof(float) * (size_t)nq * hd);
    if (attn_out) memcpy(attn_out + (int64_t)b * nq * hd, o, sizeof(float) * (size_t)nq * hd);
    if (router_out) memcpy(router_out + (int64_t)b * E, r, sizeof(float) * (size_t)E);
    if (ids_out) memcpy(ids_out + (int64_t)b * K, ids, sizeof(int32_t) * (size_t)K);
    if (w_out) memcpy(w_out + (int64_t)b * K, w, sizeof(float) * (size_t)K);
  }
  free(x); free(q); free(o); free(a); free(r); free(m); free(ids); free(w);
  free((void*)gu); free((void*)dn);
}

/* Final norm + tied LM head ("Tasks": LM_HEAD projects onto the vocabulary). */
void orc_lm_head(const orc_dims* d, int32_t batch, const float* h, const uint16_t* gamma,
                 const uint16_t* embed, float* logits) {
  const int32_t H = d->hidden;
  float* x = (float*)malloc(sizeof(float) * (size_t)H);
  for (int32_t b = 0; b < batch; ++b) {
    orc_rmsnorm(H, h + (int64_t)b * H, gamma, d->rms_eps, x);
    orc_matvec_bf16(d->vocab, H, embed, x, logits + (int64_t)b * d->vocab);
  }
  free(x);
}

void orc_decode_step(const orc_dims* d, int32_t batch, const int32_t* tokens,
                     const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                     uint16_t* kv_pool, int32_t n_pages, const uint16_t* embed,
                     const uint16_t* norm, const uint16_t* w_qkv, const uint16_t* w_o,
                     const uint16_t* w_router, const uint16_t* w_gate_up,
                     const uint16_t* w_down, float* logits, float* h_layers,
                     int32_t* ids_layers, float* w_layers) {
  const int64_t H = d->hidden, nq = d->n_q_heads, nkv = d->n_kv_heads, hd = d->head_dim;
  const int64_t E = d->n_experts, I = d->moe_inter, K = d->top_k;
  const int64_t qkv_rows = (nq + 2 * nkv) * hd;
  const int64_t kv_layer = 2 * (int64_t)n_pages * nkv * d->page_size * hd;
  float* h = (float*)malloc(sizeof(float) * (size_t)(batch * H));
  for (int32_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < H; ++i)
      h[b * H + i] = orc_bf16_to_f32(embed[(int64_t)tokens[b] * H + i]);
  for (int32_t l = 0; l < d->n_layers; ++l) {
    if (h_layers) memcpy(h_layers + (int64_t)l * batch * H, h, sizeof(float) * (size_t)(batch * H));
    /* this layer's attention window: local unless every full_every-th layer */
    orc_dims dl = *d;
    if (!(d->attn_window > 0 && (d->full_every < 1 || (l + 1) % d->full_every != 0))) dl.attn_window = 0;
    orc_layer(&dl, batch, seq_lens, page_table, max_pages, kv_pool + l * kv_layer, n_pages,
              norm + l * H, w_qkv + l * qkv_rows * H, w_o + l * H * nq * hd,
              w_router + l * E * H, w_gate_up + l * E * 2 * I * H, w_down + l * E * H * I, h,
              NULL, NULL, NULL, NULL, ids_layers ? ids_layers + (int64_t)l * batch * K : NULL,
              w_layers ? w_layers + (int64_t)l * batch * K : NULL);
  }
  if (h_layers)
    memcpy(h_layers + (int64_t)d->n_layers * batch * H, h, sizeof(float) * (size_t)(batch * H));
  orc_lm_head(d, batch, h, norm + (int64_t)d->n_layers * H, embed, logits);
  free(h);
}
