// Internal declarations shared by the C ABI glue and the HIP kernel files.
#ifndef RRA_INTERNAL_H_
#define RRA_INTERNAL_H_

#include <cstddef>
#include <cstdint>

#include "rra.h"

namespace rra {

// Largest number of blocks per row (the selection kernel holds a row in registers).
constexpr int kMaxBlocks = 4096;

// Dynamic schedule of the attention kernel: one work counter per XCD, each on
// its own 128-byte line.
constexpr int kSchedQueues = 8;
constexpr int kSchedStride = 32;  // uint32 words between counters
constexpr size_t kSchedBytes = sizeof(uint32_t) * kSchedQueues * kSchedStride;

// Device array behind rra_estimate_noalloc (one per GPU, held until exit).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

struct Shape {
  int Bz, H, Hkv, L, d, S, Bk;
  int G;   // H / Hkv
  int Ns;  // ceil(L / S)
  int Nb;  // ceil(L / Bk)
  int r;   // Bk / S, strides per block
  float scale;
  bool causal;
  // Sampled offset inside a stride for query head h: (rr_step * h + rr_shift) mod S.
  int rr_step;   // 1 for head / hybrid round-robin, 0 otherwise
  int rr_shift;  // in [0, S)
};

Shape shape_of(const rra_params_t& p);
size_t kagg_bytes(const Shape& s);
size_t score_bytes(const Shape& s);
size_t align_up(size_t x, size_t a);

// Kernel launchers (defined in kernels/*.hip).  They return the value of
// hipGetLastError() after the launch, as an int (0 = success).
int launch_cast_f32_bf16(const float* src, uint16_t* dst, int64_t n, void* stream);
int launch_stride_aggregate(const Shape& s, const uint16_t* k, uint16_t* kagg, void* stream);
int launch_block_scores(const Shape& s, const uint16_t* q, const uint16_t* kagg, float* score,
                        void* stream);
int launch_top_tau(const Shape& s, float tau, int protect_last, const float* score, uint8_t* mask,
                   int32_t* idx, int32_t* cnt, void* stream);
int launch_xattn_scores(const Shape& s, const uint16_t* q, const uint16_t* k, float* score, void* stream);
int launch_block_mass(const Shape& s, const uint16_t* q, const uint16_t* k, float* mass, void* stream);
// sched: kSchedBytes of device memory for the dynamic schedule, or nullptr
// for one workgroup per (b, h, I) row.
int launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* idx, const int32_t* cnt, uint16_t* out, uint32_t* sched, void* stream);

}  // namespace rra

#endif  // RRA_INTERNAL_H_
