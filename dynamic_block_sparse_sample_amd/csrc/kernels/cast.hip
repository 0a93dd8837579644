// float32 -> bfloat16 conversion, round to nearest even.  Streams 32 bytes in
// and 16 bytes out per thread; HBM-bound.
#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

__global__ __launch_bounds__(256) void cast_f32_bf16_kernel(const float* __restrict__ src,
                                                            uint16_t* __restrict__ dst, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i + 8 <= n) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(src + i);
    const floatx4 b = *reinterpret_cast<const floatx4*>(src + i + 4);
    u32x4 o;
    o[0] = pack_bf16x2(a[0], a[1]);
    o[1] = pack_bf16x2(a[2], a[3]);
    o[2] = pack_bf16x2(b[0], b[1]);
    o[3] = pack_bf16x2(b[2], b[3]);
    *reinterpret_cast<u32x4*>(dst + i) = o;
  } else {
    for (int64_t j = i; j < n; ++j) {
      __bf16 h = static_cast<__bf16>(src[j]);
      dst[j] = __builtin_bit_cast(uint16_t, h);
    }
  }
}

int launch_cast_f32_bf16(const float* src, uint16_t* dst, int64_t n, void* stream) {
  if (n <= 0) return 0;
  const int64_t blocks = (n + 2047) / 2048;
  hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), src, dst, n);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
