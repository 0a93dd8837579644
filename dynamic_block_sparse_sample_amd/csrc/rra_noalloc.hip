// rra_estimate_noalloc: the whole estimator with its intermediates (the
// aggregated keys and, when the caller passes no score buffer, the block
// scores) in a file-scope device array instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array is a static __device__ object: every GPU the library runs on holds
// one copy of kNoAllocScratchBytes until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); the device address comes from hipGetSymbolAddress, taken once
// per device with that device current and cached here.  Calls on one GPU share
// its array, so calls that overlap in time on one GPU (two streams, or two
// host threads) race on it; the estimator's kernels overwrite every byte they
// later read, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "rra.h"
#include "rra_internal.h"

namespace rra {

static_assert(kNoAllocScratchBytes == RRA_NOALLOC_SCRATCH_BYTES, "header and library agree on the limit");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of this device's copy of `scratch`, or nullptr on a HIP error.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    ptr = p;
  }
  return ptr;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace rra

extern "C" {

rra_status_t rra_estimate_noalloc(const rra_params_t* p, const void* q, const void* k, uint8_t* mask, int32_t* idx,
                                  int32_t* cnt, float* score, void* stream) {
  rra_status_t st = rra_validate(p);
  if (st != RRA_OK) return st;
  if (p->batch == 0 || p->seq_len == 0) return RRA_OK;
  if (q == nullptr || k == nullptr || mask == nullptr || idx == nullptr || cnt == nullptr) return RRA_ERR_INVALID_ARG;
  if (!rra::aligned16(q) || !rra::aligned16(k) || !rra::aligned16(idx) || !rra::aligned16(cnt))
    return RRA_ERR_INVALID_ARG;
  if (score != nullptr && !rra::aligned16(score)) return RRA_ERR_INVALID_ARG;
  const rra::Shape s = rra::shape_of(*p);
  const size_t kagg_at = 0;
  const size_t score_at = rra::align_up(rra::kagg_bytes(s), 256);
  const size_t need = score != nullptr ? rra::kagg_bytes(s) : score_at + rra::score_bytes(s);
  if (need > rra::kNoAllocScratchBytes) return RRA_ERR_WORKSPACE;
  uint8_t* base = static_cast<uint8_t*>(rra::scratch_on_current_device());
  if (base == nullptr) return RRA_ERR_HIP;
  uint16_t* kagg = reinterpret_cast<uint16_t*>(base + kagg_at);
  float* sc = score != nullptr ? score : reinterpret_cast<float*>(base + score_at);
  int err = rra::launch_stride_aggregate(s, static_cast<const uint16_t*>(k), kagg, stream);
  if (err == 0) err = rra::launch_block_scores(s, static_cast<const uint16_t*>(q), kagg, sc, stream);
  if (err == 0) err = rra::launch_top_tau(s, p->tau, p->protect_last, sc, mask, idx, cnt, stream);
  return err == 0 ? RRA_OK : RRA_ERR_HIP;
}

}  // extern "C"
