// mkd_static.hip - the decode step for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// mkd_decode_step_static runs the same step as mkd_decode_step with the engine's
// workspace in a library-owned static device array instead of a caller buffer.
//
// The array is a file-scope __device__ variable.  Host code cannot use its name as a
// device address, so its address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; only that address is
// passed to kernels and copies.  Every call on one GPU shares that GPU's array, which
// keeps the last call's contents: a call from an engine other than the last one to use
// it clears the array and copies the engine's schedule in first (in order on the
// caller's stream), and the tagged words' step epoch continues per array.  Calls that
// overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mkd.h"

namespace mkd {
int check_step_state(mkd_engine* e);
int enqueue_step(mkd_engine* e, char* ws, uint32_t* epoch, void* stream, int32_t batch, const int32_t* d_tokens,
                 const int32_t* d_seq_lens, const int32_t* h_seq_lens, const int32_t* d_page_table,
                 const int32_t* h_page_table, void* kv_pool, int32_t n_pages, float* d_logits);
hipError_t init_workspace(const mkd_engine* e, char* ws, hipStream_t stream);
uint64_t engine_id(const mkd_engine* e);
int32_t engine_device(const mkd_engine* e);
size_t engine_ws_bytes(const mkd_engine* e);
int engine_fail(mkd_engine* e, int code, const char* msg);
}  // namespace mkd

static __device__ __align__(256) unsigned char scratch[MKD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  char* ptr = nullptr;   // device address of `scratch` on this device (hipGetSymbolAddress)
  uint64_t owner = 0;    // id of the engine whose schedule the array holds (0: none)
  uint32_t epoch = 0;    // step epoch of the last step run in the array
};

std::mutex g_mutex;
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

extern "C" int mkd_decode_step_static(mkd_engine* e, void* stream, int32_t batch, const int32_t* d_tokens,
                                      const int32_t* d_seq_lens, const int32_t* h_seq_lens,
                                      const int32_t* d_page_table, const int32_t* h_page_table, void* kv_pool,
                                      int32_t n_pages, float* d_logits) {
  using namespace mkd;
  if (!e) return MKD_ERR_ARG;
  const int st = check_step_state(e);
  if (st != MKD_OK) return st;
  const int dev = engine_device(e);
  if (dev >= kMaxDevices) return engine_fail(e, MKD_ERR_ARG, "device index beyond the static scratch table");
  if (engine_ws_bytes(e) > (size_t)MKD_STATIC_SCRATCH_BYTES)
    return engine_fail(e, MKD_ERR_CAPACITY,
                       "the engine's workspace (mkd_workspace_bytes) exceeds MKD_STATIC_SCRATCH_BYTES; use "
                       "mkd_decode_step with a caller workspace, or a smaller max_batch / max_pages_per_seq");
  std::lock_guard<std::mutex> lock(g_mutex);
  hipError_t rc = hipSetDevice(dev);
  if (rc != hipSuccess) return engine_fail(e, MKD_ERR_HIP, "hipSetDevice failed");
  DeviceScratch& d = g_scratch[dev];
  if (!d.ptr) {
    void* addr = nullptr;
    rc = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (rc != hipSuccess || !addr) return engine_fail(e, MKD_ERR_HIP, "hipGetSymbolAddress of the static scratch failed");
    d.ptr = (char*)addr;
  }
  if (d.owner != engine_id(e)) {
    d.owner = 0;
    rc = init_workspace(e, d.ptr, (hipStream_t)stream);
    if (rc != hipSuccess) return engine_fail(e, MKD_ERR_HIP, "static scratch initialisation failed");
    d.owner = engine_id(e);
    d.epoch = 0;
  }
  return enqueue_step(e, d.ptr, &d.epoch, stream, batch, d_tokens, d_seq_lens, h_seq_lens, d_page_table,
                      h_page_table, kv_pool, n_pages, d_logits);
}
