// mkd_serve.hip - the continuous-decode loop around the step (section "The serving engine
// around the kernel": per step the host updates the KV positions and page tables, clears
// the step state, selects the schedule by the live context and launches; sampling and
// retirement follow, and sequences join and finish between steps).
//
// The server owns the host side of a ragged batch: a free list of KV-cache pages, the
// live sequences in join order (cached length, tokens still to generate, pages), and a
// small device buffer the caller provides (inputs of the step, logits, sampled tokens).
// A step schedules the live sequences in join order up to the engine's max_batch.  A
// sequence whose next token starts a new page takes one from the free list; when the
// list is empty it is parked (it keeps its pages and is not scheduled) and resumes at the
// first step where a page is free.  After the step kernel two argmax kernels sample every
// row (ties to the lower token id) into the token that sequence is fed next; sequences
// that have generated their tokens retire and return their pages.  The step's attention
// item size follows the longest live context (chosen inside the engine's step).
//
// Per step the host makes one asynchronous upload (lengths, page-table rows, sequence
// slots, first tokens of new sequences) from one of two pinned staging buffers and one
// asynchronous download of the fed and sampled tokens; it allocates nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mkd.h"

namespace mkd {
int32_t engine_device(const mkd_engine* e);
void engine_limits(const mkd_engine* e, int32_t* max_batch, int32_t* max_pages, int32_t* vocab, int32_t* page);
}  // namespace mkd

namespace {

// tokens[b]: the first token of a new sequence, else the token sampled for its slot
__global__ void serve_gather(const int32_t* __restrict__ slot_of, const int32_t* __restrict__ join_tok,
                             const int32_t* __restrict__ slot_tok, int32_t* __restrict__ tokens, int32_t batch) {
  const int b = threadIdx.x;
  if (b < batch) {
    const int32_t j = join_tok[b];
    tokens[b] = j >= 0 ? j : slot_tok[slot_of[b]];
  }
}

// Greedy sampling in two passes: workgroup (c, b) finds the largest logit of chunk c of
// row b (kArgmaxChunks chunks per row, 256 threads) and its lowest index among equal
// maxima; one wave per row then combines the chunks in the same way.  NaN never wins; a
// row without a number gives token 0.
constexpr int kArgmaxChunks = 64;

__device__ __forceinline__ void argmax_take(float& best, int32_t& bi, float v, int32_t i) {
  if (v > best || (v == best && i < bi)) {
    best = v;
    bi = i;
  }
}
__device__ __forceinline__ void argmax_wave(float& best, int32_t& bi) {
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int32_t oi = __shfl_xor(bi, off);
    argmax_take(best, bi, ov, oi);
  }
}

__global__ void __launch_bounds__(256) serve_argmax_chunks(const float* __restrict__ logits, int32_t vocab,
                                                           float* __restrict__ part_v, int32_t* __restrict__ part_i) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int per = (vocab + kArgmaxChunks - 1) / kArgmaxChunks;
  const int lo = c * per, hi = min(vocab, lo + per);
  const float* row = logits + (int64_t)b * vocab;
  float best = -INFINITY;
  int32_t bi = 0x7FFFFFFF;
  for (int i = lo + (int)threadIdx.x; i < hi; i += 256) argmax_take(best, bi, row[i], i);
  argmax_wave(best, bi);
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = best;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) argmax_take(best, bi, sv[w], si[w]);
    part_v[b * kArgmaxChunks + c] = best;
    part_i[b * kArgmaxChunks + c] = bi;
  }
}

__global__ void __launch_bounds__(64) serve_argmax_final(const float* __restrict__ part_v, const int32_t* __restrict__ part_i,
                                                         const int32_t* __restrict__ slot_of, int32_t* __restrict__ slot_tok,
                                                         int32_t* __restrict__ sampled) {
  const int b = blockIdx.x;
  float best = part_v[b * kArgmaxChunks + threadIdx.x];
  int32_t bi = part_i[b * kArgmaxChunks + threadIdx.x];
  argmax_wave(best, bi);
  if (threadIdx.x == 0) {
    if (bi == 0x7FFFFFFF) bi = 0;
    sampled[b] = bi;
    slot_tok[slot_of[b]] = bi;
  }
}
static_assert(kArgmaxChunks == 64, "the final pass is one wave");

struct Seq {
  int64_t id;
  int32_t len;        // cached tokens; the next token is fed at this position
  int32_t remaining;  // tokens still to generate
  int32_t slot;       // index into the per-slot sampled-token array
  int32_t first_token;
  bool fresh;         // not yet stepped: fed first_token
  bool parked;
  std::vector<int32_t> pages;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct mkd_server {
  mkd_engine* eng = nullptr;
  int32_t device = -1, n_pages = 0, max_live = 0, max_batch = 0, max_pages = 0, vocab = 0, page = 0;
  std::vector<int32_t> free_pages;  // a stack; the lowest page on top at creation
  std::vector<Seq> live;            // join order
  std::vector<char> slot_used;
  // device buffer (caller-owned): upload area | tokens | per-slot tokens | sampled |
  // argmax partials | logits
  char* dev = nullptr;
  size_t off_up = 0, off_tok = 0, off_slot = 0, off_smp = 0, off_part = 0, off_logits = 0, bytes = 0;
  int32_t up_ints = 0;  // 3 * max_batch + max_batch * max_pages
  // pinned host memory: two staging copies of the upload area, fed and sampled tokens
  int32_t* stage[2] = {nullptr, nullptr};
  int32_t* h_fed = nullptr;
  int32_t* h_smp = nullptr;
  hipEvent_t ev_stage[2] = {nullptr, nullptr};
  bool stage_pending[2] = {false, false};
  int cur = 0;
  // the last step
  int32_t last_batch = 0;
  hipStream_t last_stream = nullptr;
  std::vector<int64_t> last_ids;
  std::vector<int32_t> last_lens, last_table;
  std::string err;
  // a server over a host-only engine does the bookkeeping of every step without
  // launching anything (the scheduling logic, testable without a GPU)
  bool dry = false;
  std::vector<int32_t> dry_stage;
  std::vector<int32_t> dry_fed;
};

namespace {
int sfail(mkd_server* s, int code, const std::string& msg) {
  s->err = msg;
  return code;
}
int shfail(mkd_server* s, hipError_t rc, const char* what) {
  return sfail(s, MKD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(rc));
}
}  // namespace

extern "C" {

int mkd_server_create(mkd_engine* eng, int32_t n_pages, int32_t max_live, mkd_server** out) {
  if (!out) return MKD_ERR_ARG;
  *out = nullptr;
  if (!eng || n_pages < 1 || max_live < 1 || max_live > 4096) return MKD_ERR_ARG;
  mkd_server* s = new mkd_server();
  s->eng = eng;
  s->device = mkd::engine_device(eng);
  s->dry = s->device < 0;
  s->n_pages = n_pages;
  s->max_live = max_live;
  mkd::engine_limits(eng, &s->max_batch, &s->max_pages, &s->vocab, &s->page);
  s->free_pages.resize(n_pages);
  for (int32_t i = 0; i < n_pages; ++i) s->free_pages[i] = n_pages - 1 - i;
  s->slot_used.assign(max_live, 0);
  s->up_ints = 3 * s->max_batch + s->max_batch * s->max_pages;
  size_t at = 0;
  s->off_up = at;
  at = align256(at + sizeof(int32_t) * (size_t)s->up_ints);
  s->off_tok = at;
  at = align256(at + sizeof(int32_t) * (size_t)s->max_batch);
  s->off_slot = at;
  at = align256(at + sizeof(int32_t) * (size_t)max_live);
  s->off_smp = at;
  at = align256(at + sizeof(int32_t) * (size_t)s->max_batch);
  s->off_part = at;
  at = align256(at + (sizeof(float) + sizeof(int32_t)) * (size_t)s->max_batch * kArgmaxChunks);
  s->off_logits = at;
  at = align256(at + sizeof(float) * (size_t)s->max_batch * s->vocab);
  s->bytes = at;
  if (s->dry) {
    s->dry_stage.resize(s->up_ints);
    s->dry_fed.resize(s->max_batch);
    *out = s;
    return MKD_OK;
  }
  hipError_t rc = hipSetDevice(s->device);
  for (int k = 0; k < 2 && rc == hipSuccess; ++k) {
    rc = hipHostMalloc((void**)&s->stage[k], sizeof(int32_t) * (size_t)s->up_ints, hipHostMallocDefault);
    if (rc == hipSuccess) rc = hipEventCreateWithFlags(&s->ev_stage[k], hipEventDisableTiming);
  }
  if (rc == hipSuccess) rc = hipHostMalloc((void**)&s->h_fed, sizeof(int32_t) * (size_t)s->max_batch, hipHostMallocDefault);
  if (rc == hipSuccess) rc = hipHostMalloc((void**)&s->h_smp, sizeof(int32_t) * (size_t)s->max_batch, hipHostMallocDefault);
  if (rc != hipSuccess) {
    mkd_server_destroy(s);
    return MKD_ERR_HIP;
  }
  *out = s;
  return MKD_OK;
}

void mkd_server_destroy(mkd_server* s) {
  if (!s) return;
  if (s->dry) {
    delete s;
    return;
  }
  (void)hipSetDevice(s->device);
  for (int k = 0; k < 2; ++k) {
    if (s->ev_stage[k]) {
      (void)hipEventSynchronize(s->ev_stage[k]);
      (void)hipEventDestroy(s->ev_stage[k]);
    }
    if (s->stage[k]) (void)hipHostFree(s->stage[k]);
  }
  if (s->last_stream) (void)hipStreamSynchronize(s->last_stream);
  if (s->h_fed) (void)hipHostFree(s->h_fed);
  if (s->h_smp) (void)hipHostFree(s->h_smp);
  delete s;
}

size_t mkd_server_buffer_bytes(const mkd_server* s) { return s && !s->dry ? s->bytes : 0; }

int mkd_server_set_buffer(mkd_server* s, void* dev_ptr, size_t bytes) {
  if (!s) return MKD_ERR_ARG;
  if (s->dry) return sfail(s, MKD_ERR_STATE, "a server over a host-only engine has no device buffer");
  if (!dev_ptr || ((uintptr_t)dev_ptr & 255)) return sfail(s, MKD_ERR_ARG, "buffer must be non-NULL and 256-byte aligned");
  if (bytes < s->bytes) return sfail(s, MKD_ERR_ARG, "buffer smaller than mkd_server_buffer_bytes");
  if (!s->live.empty()) return sfail(s, MKD_ERR_STATE, "sequences are live");
  s->dev = (char*)dev_ptr;
  return MKD_OK;
}

int mkd_server_join(mkd_server* s, int64_t seq_id, int32_t cached_len, int32_t first_token, int32_t max_new_tokens,
                    int32_t* h_pages, int32_t max_pages_out) {
  if (!s) return MKD_ERR_ARG;
  if (cached_len < 0 || max_new_tokens < 1 || first_token < 0 || first_token >= s->vocab)
    return sfail(s, MKD_ERR_ARG, "cached_len >= 0, max_new_tokens >= 1 and first_token in [0, vocab) are required");
  // the last token fed sits at position cached_len + max_new_tokens - 1
  const int64_t last_pos = (int64_t)cached_len + max_new_tokens - 1;
  if (last_pos / s->page >= s->max_pages) return sfail(s, MKD_ERR_ARG, "sequence longer than max_pages_per_seq pages");
  for (const Seq& q : s->live)
    if (q.id == seq_id) return sfail(s, MKD_ERR_ARG, "sequence id already live");
  if ((int32_t)s->live.size() >= s->max_live) return sfail(s, MKD_ERR_CAPACITY, "max_live sequences are live");
  const int32_t need = (cached_len + s->page - 1) / s->page;
  if (need > (int32_t)s->free_pages.size()) return sfail(s, MKD_ERR_CAPACITY, "not enough free KV pages");
  if (need > 0 && (!h_pages || max_pages_out < need)) return sfail(s, MKD_ERR_ARG, "h_pages too small");
  Seq q;
  q.id = seq_id;
  q.len = cached_len;
  q.remaining = max_new_tokens;
  q.first_token = first_token;
  q.fresh = true;
  q.parked = false;
  q.slot = (int32_t)(std::find(s->slot_used.begin(), s->slot_used.end(), 0) - s->slot_used.begin());
  s->slot_used[q.slot] = 1;
  for (int32_t i = 0; i < need; ++i) {
    q.pages.push_back(s->free_pages.back());
    s->free_pages.pop_back();
    h_pages[i] = q.pages.back();
  }
  s->live.push_back(std::move(q));
  return MKD_OK;
}

int mkd_server_step(mkd_server* s, void* stream, void* kv_pool, int32_t* n_scheduled) {
  if (!s || !n_scheduled) return MKD_ERR_ARG;
  *n_scheduled = 0;
  if (!s->dry && !s->dev) return sfail(s, MKD_ERR_STATE, "no device buffer (mkd_server_set_buffer)");
  if (!s->dry && !kv_pool) return sfail(s, MKD_ERR_ARG, "kv_pool is NULL");
  if (s->live.empty()) {
    s->last_batch = 0;
    return MKD_OK;
  }
  // schedule: join order, up to max_batch; a sequence whose next token opens a page
  // takes one from the free list or is parked
  std::vector<Seq*> batch;
  for (Seq& q : s->live) {
    if ((int32_t)batch.size() == s->max_batch) break;
    if (q.len / s->page >= (int32_t)q.pages.size()) {
      if (s->free_pages.empty()) {
        q.parked = true;
        continue;
      }
      q.pages.push_back(s->free_pages.back());
      s->free_pages.pop_back();
    }
    q.parked = false;
    batch.push_back(&q);
  }
  const int32_t B = (int32_t)batch.size();
  if (B == 0) return sfail(s, MKD_ERR_CAPACITY, "every live sequence is parked: the KV pool has no free page");
  hipError_t rc = s->dry ? hipSuccess : hipSetDevice(s->device);
  if (rc != hipSuccess) return shfail(s, rc, "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  // staging copy `cur` is free once the upload that last read it has completed
  if (!s->dry && s->stage_pending[s->cur]) {
    rc = hipEventSynchronize(s->ev_stage[s->cur]);
    if (rc != hipSuccess) return shfail(s, rc, "staging wait");
    s->stage_pending[s->cur] = false;
  }
  int32_t* up = s->dry ? s->dry_stage.data() : s->stage[s->cur];
  const int32_t MB = s->max_batch, MP = s->max_pages;
  int32_t* lens = up;
  int32_t* slot_of = up + MB;
  int32_t* join = up + 2 * MB;
  int32_t* table = up + 3 * MB;
  for (int32_t b = 0; b < B; ++b) {
    const Seq& q = *batch[b];
    lens[b] = q.len;
    slot_of[b] = q.slot;
    join[b] = q.fresh ? q.first_token : -1;
    int32_t* row = table + (size_t)b * MP;
    std::copy(q.pages.begin(), q.pages.end(), row);
    std::fill(row + q.pages.size(), row + MP, -1);
  }
  if (s->dry) {
    for (int32_t b = 0; b < B; ++b) s->dry_fed[b] = join[b];  // a sampled token is unknown: -1
  } else {
  int32_t* d_up = (int32_t*)(s->dev + s->off_up);
  int32_t* d_tok = (int32_t*)(s->dev + s->off_tok);
  int32_t* d_slot = (int32_t*)(s->dev + s->off_slot);
  int32_t* d_smp = (int32_t*)(s->dev + s->off_smp);
  float* d_logits = (float*)(s->dev + s->off_logits);
  const size_t up_bytes = sizeof(int32_t) * (3 * (size_t)MB + (size_t)B * MP);
  rc = hipMemcpyAsync(d_up, up, up_bytes, hipMemcpyHostToDevice, st);
  if (rc == hipSuccess) rc = hipEventRecord(s->ev_stage[s->cur], st);
  if (rc != hipSuccess) return shfail(s, rc, "upload");
  s->stage_pending[s->cur] = true;
  serve_gather<<<1, 64, 0, st>>>(d_up + MB, d_up + 2 * MB, d_slot, d_tok, B);
  rc = hipGetLastError();
  if (rc != hipSuccess) return shfail(s, rc, "token gather launch");
  const int r = mkd_decode_step(s->eng, stream, B, d_tok, d_up, lens, d_up + 3 * MB, table, kv_pool, s->n_pages, d_logits);
  if (r != MKD_OK) return sfail(s, r, std::string("step: ") + mkd_last_error(s->eng));
  float* d_pv = (float*)(s->dev + s->off_part);
  int32_t* d_pi = (int32_t*)(d_pv + (size_t)MB * kArgmaxChunks);
  serve_argmax_chunks<<<dim3(kArgmaxChunks, B), 256, 0, st>>>(d_logits, s->vocab, d_pv, d_pi);
  rc = hipGetLastError();
  if (rc == hipSuccess) {
    serve_argmax_final<<<B, 64, 0, st>>>(d_pv, d_pi, d_up + MB, d_slot, d_smp);
    rc = hipGetLastError();
  }
  if (rc == hipSuccess) rc = hipMemcpyAsync(s->h_fed, d_tok, sizeof(int32_t) * B, hipMemcpyDeviceToHost, st);
  if (rc == hipSuccess) rc = hipMemcpyAsync(s->h_smp, d_smp, sizeof(int32_t) * B, hipMemcpyDeviceToHost, st);
  if (rc != hipSuccess) return shfail(s, rc, "sampling");
  }
  // the step as scheduled, then advance and retire
  s->last_batch = B;
  s->last_stream = st;
  s->last_ids.resize(B);
  s->last_lens.assign(lens, lens + B);
  s->last_table.assign(table, table + (size_t)B * MP);
  for (int32_t b = 0; b < B; ++b) {
    Seq& q = *batch[b];
    s->last_ids[b] = q.id;
    q.len += 1;
    q.remaining -= 1;
    q.fresh = false;
  }
  for (size_t i = 0; i < s->live.size();) {
    Seq& q = s->live[i];
    if (q.remaining == 0) {
      // pages go back in reverse, so the sequence's first page is the next one handed out
      for (auto it = q.pages.rbegin(); it != q.pages.rend(); ++it) s->free_pages.push_back(*it);
      s->slot_used[q.slot] = 0;
      s->live.erase(s->live.begin() + (ptrdiff_t)i);
    } else {
      ++i;
    }
  }
  s->cur ^= 1;
  *n_scheduled = B;
  return MKD_OK;
}

int mkd_server_last_step(mkd_server* s, int64_t* ids, int32_t* fed, int32_t* sampled, int32_t* seq_lens,
                         int32_t* page_table, float* logits, int32_t max_batch_out, int32_t* batch) {
  if (!s || !batch) return MKD_ERR_ARG;
  *batch = s->last_batch;
  if (s->last_batch == 0) return MKD_OK;
  if (max_batch_out < s->last_batch) return sfail(s, MKD_ERR_CAPACITY, "max_batch_out too small");
  hipError_t rc = s->dry ? hipSuccess : hipSetDevice(s->device);
  if (rc == hipSuccess && !s->dry) rc = hipStreamSynchronize(s->last_stream);
  if (rc != hipSuccess) return shfail(s, rc, "synchronise");
  const int32_t B = s->last_batch;
  if (ids) std::copy(s->last_ids.begin(), s->last_ids.end(), ids);
  if (fed) std::memcpy(fed, s->dry ? s->dry_fed.data() : s->h_fed, sizeof(int32_t) * B);
  if (sampled) {
    if (s->dry) std::fill(sampled, sampled + B, -1);
    else std::memcpy(sampled, s->h_smp, sizeof(int32_t) * B);
  }
  if (seq_lens) std::copy(s->last_lens.begin(), s->last_lens.end(), seq_lens);
  if (page_table) std::copy(s->last_table.begin(), s->last_table.end(), page_table);
  if (logits) {
    if (s->dry) return sfail(s, MKD_ERR_STATE, "a server over a host-only engine has no logits");
    rc = hipMemcpy(logits, s->dev + s->off_logits, sizeof(float) * (size_t)B * s->vocab, hipMemcpyDeviceToHost);
    if (rc != hipSuccess) return shfail(s, rc, "logits copy");
  }
  return MKD_OK;
}

int mkd_server_stats(const mkd_server* s, int32_t* n_live, int32_t* n_parked, int32_t* n_free_pages) {
  if (!s) return MKD_ERR_ARG;
  int32_t parked = 0;
  for (const Seq& q : s->live) parked += q.parked ? 1 : 0;
  if (n_live) *n_live = (int32_t)s->live.size();
  if (n_parked) *n_parked = parked;
  if (n_free_pages) *n_free_pages = (int32_t)s->free_pages.size();
  return MKD_OK;
}

const char* mkd_server_last_error(const mkd_server* s) { return s ? s->err.c_str() : ""; }

}  // extern "C"
