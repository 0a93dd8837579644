// Direct global-to-LDS copies of 16-byte chunks into rows whose chunks are
// XOR-swizzled, shared by the attention and block-score kernels.
#ifndef RRA_LDS_COPY_H_
#define RRA_LDS_COPY_H_

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rra {

// Chunk swizzle of key row r (bits: r1 -> 3, r0 -> 2, r1^r3 -> 1, r2 -> 0).
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 3) | ((r & 1) << 2) | ((((r >> 1) ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane from global memory (gbase + voff) into LDS at
// lds + OFF + 16 * lane (global_load_lds_dwordx4, saddr form).  Issued from
// inline asm so that the compiler does not tie later LDS reads of the other
// pipeline stage to this copy with a full vmcnt wait; completion is tracked
// explicitly with wait_vmcnt.  m0 (the LDS address) is formed from one base
// register and an immediate, so the copies of a tile share one SGPR, and is
// saved and restored.
template <int OFF>
__device__ __forceinline__ void copy16_to_lds(const uint8_t* gbase, int voff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %3, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds), "i"(OFF)
      : "memory", "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

}  // namespace rra

#endif  // RRA_LDS_COPY_H_
