// mkd_litmus.hip - message-passing litmus test of the step's inter-workgroup protocol
// (section "Barriers": producers publish, consumers spin until the dependency is met; the
// fences must leave no data race across SMs - here across XCDs, whose L2 caches are not
// coherent with each other).
//
// Workgroups 2p and 2p + 1 (one wave each; workgroup w runs on XCD w mod 8, so the two
// sit on different XCDs) form a producer / consumer pair and run `rounds` rounds over the
// same buffers, as the step reuses its buffers across layers and steps:
//   tagged words   the producer stores 256 tagged words (value, round) with the step's
//                  agent-scope 64-bit stores; the consumer polls each with agent-scope
//                  loads until its tag is the round and checks its value: a word whose tag
//                  is new but whose value is old would be a torn or reordered word;
//   flag and data  the producer stores 512 bf16 data words with the agent-scope 16-bit
//                  stores that write the new token's K/V, waits for them, then stores a
//                  tagged flag, as a QKV tile raises its K/V flag; the consumer polls the
//                  flag, acquires at agent scope and reads the data with the non-temporal
//                  16-byte loads that read K/V pages: a stale value means the acquire or
//                  the producer's wait does not order the data;
// then the consumer acknowledges the round with a tagged word, and the producer waits for
// the acknowledgement before the next round.  Every wait is bounded; a workgroup stops at
// its first timeout, so the kernel always ends.
#include <hip/hip_runtime.h>

#include "../../include/mkd.h"
#include "mkd_device.h"

namespace {
using namespace mkd;

constexpr int kWords = 256;  // tagged words per pair (4 per lane)
constexpr int kData = 512;   // bf16 data words per pair (8 per lane)

__device__ __forceinline__ float word_value(int r, int i) { return (float)(r * 1000 + i); }
__device__ __forceinline__ uint16_t data_value(int r, int i) { return (uint16_t)((r * 131 + i * 7) & 0xFFFF); }

__global__ void __launch_bounds__(64) litmus_kernel(uint64_t* words, uint16_t* data, uint64_t* flags, uint64_t* acks,
                                                   int32_t rounds, int32_t spin_limit, uint32_t* result) {
  const int pair = blockIdx.x >> 1, consumer = blockIdx.x & 1, lane = threadIdx.x;
  GAS uint64_t* w = gas(words) + (int64_t)pair * kWords;
  GAS uint16_t* d = gas(data) + (int64_t)pair * kData;
  GAS uint64_t* flag = gas(flags) + pair;
  GAS uint64_t* ack = gas(acks) + pair;
  uint32_t torn = 0, stale = 0, timeouts = 0, done = 0;
  // waits until every lane's word at p (one per lane, or lane 0's) carries tag r
  auto wait_tag = [&](const GAS uint64_t* p, bool per_lane, uint32_t r, uint64_t& v) -> bool {
    v = ld_tag(per_lane ? p + lane : p);
    int32_t spins = 0;
    while (__ballot(!tag_is(v, r)) != 0) {
      if (++spins > spin_limit) return false;
      __builtin_amdgcn_s_sleep(1);
      if (!tag_is(v, r)) v = ld_tag(per_lane ? p + lane : p);
    }
    return true;
  };
  for (int r = 1; r <= rounds; ++r) {
    const uint32_t tag = (uint32_t)r;
    if (!consumer) {
      for (int u = 0; u < kWords / 64; ++u) st_tag(w + u * 64 + lane, word_value(r, u * 64 + lane), tag);
      for (int u = 0; u < kData / 64; ++u) st_pub(d + u * 64 + lane, data_value(r, u * 64 + lane));
      wait_vm_all();
      if (lane == 0) st_tag(flag, 0.0f, tag);
      uint64_t v;
      if (!wait_tag(ack, false, tag, v)) {
        ++timeouts;
        break;
      }
    } else {
      bool ok = true;
      for (int u = 0; u < kWords / 64 && ok; ++u) {
        uint64_t v;
        ok = wait_tag(w + u * 64, true, tag, v);
        if (ok && tag_val(v) != word_value(r, u * 64 + lane)) ++torn;
      }
      uint64_t f;
      if (ok) ok = wait_tag(flag, false, tag, f);
      if (!ok) {
        ++timeouts;
        break;
      }
      fence_acquire_agent();
      const u32x4 q = ld_stream16(d + lane * 8);
      const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
      for (int e = 0; e < 8; ++e) {
        const uint16_t got = (uint16_t)(qq[e / 2] >> (16 * (e & 1)));
        if (got != data_value(r, lane * 8 + e)) ++stale;
      }
      if (lane == 0) st_tag(ack, 0.0f, tag);
    }
    ++done;
  }
  // per-lane counts summed into the result with vector atomics
  if (torn) atomicAdd(result + 0, torn);
  if (stale) atomicAdd(result + 1, stale);
  if (lane == 0 && timeouts) atomicAdd(result + 2, timeouts);
  if (lane == 0 && consumer) atomicAdd(result + 3, done);
}

}  // namespace

extern "C" int mkd_protocol_litmus(int32_t hip_device, int32_t n_pairs, int32_t rounds, uint32_t* h_result) {
  if (!h_result || n_pairs < 1 || n_pairs > 4096 || rounds < 1 || rounds > 100000) return MKD_ERR_ARG;
  hipError_t rc = hipSetDevice(hip_device);
  if (rc != hipSuccess) return MKD_ERR_HIP;
  const size_t bw = sizeof(uint64_t) * (size_t)n_pairs * kWords, bd = sizeof(uint16_t) * (size_t)n_pairs * kData;
  const size_t bf = sizeof(uint64_t) * (size_t)n_pairs, br = 4 * sizeof(uint32_t);
  char* buf = nullptr;
  rc = hipMalloc(&buf, bw + bd + 2 * bf + br);
  if (rc != hipSuccess) return MKD_ERR_HIP;
  // tag 0 everywhere: no round has been published
  rc = hipMemset(buf, 0, bw + bd + 2 * bf + br);
  uint64_t* words = (uint64_t*)buf;
  uint16_t* data = (uint16_t*)(buf + bw);
  uint64_t* flags = (uint64_t*)(buf + bw + bd);
  uint64_t* acks = flags + n_pairs;
  uint32_t* result = (uint32_t*)(buf + bw + bd + 2 * bf);
  int32_t spin_limit = 2000000;
  if (rc == hipSuccess) {
    void* args[] = {&words, &data, &flags, &acks, &rounds, &spin_limit, &result};
    rc = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&litmus_kernel), dim3(2 * n_pairs), dim3(64),
                                    args, 0, nullptr);
  }
  if (rc == hipSuccess) rc = hipDeviceSynchronize();
  if (rc == hipSuccess) rc = hipMemcpy(h_result, result, br, hipMemcpyDeviceToHost);
  (void)hipFree(buf);
  return rc == hipSuccess ? MKD_OK : MKD_ERR_HIP;
}
