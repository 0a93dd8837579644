// Stride key aggregation (RRAttention §3.2): the key vectors of each stride of
// S tokens are summed, divided by S and rounded once to bfloat16.  A last
// partial stride (L not a multiple of S) sums the keys it has, still times 1/S.
//
// One thread owns 8 channels (16 bytes) of one stride; 16 consecutive threads
// cover a 256-byte key row, so every load instruction reads whole rows.  The
// sum of S bf16 values is exact in float64; the float64 -> bf16 rounding goes
// through float32 with round-to-odd, which gives the correctly rounded bf16
// result (float32 keeps 24 >= 8 + 2 bits).  HBM-bound: reads K once, writes
// Kagg (1/S of K).
#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

// float64 -> float32 rounded to odd: truncate toward zero, then set the last
// bit if anything was discarded.
__device__ __forceinline__ float f64_to_f32_round_odd(double x) {
  float f = static_cast<float>(x);  // round to nearest
  const double back = static_cast<double>(f);
  if (back != x) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(x)) u -= 1;  // rounded away from zero: step back toward zero
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f;
}

template <int D>
__global__ __launch_bounds__(256) void stride_aggregate_kernel(const uint16_t* __restrict__ k,
                                                               uint16_t* __restrict__ kagg,
                                                               int rows, int S, int Ns, int L, double inv_s) {
  constexpr int CH = D / 8;  // 16-byte chunks per key row
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int row = static_cast<int>(gid / CH);  // (b, g, j) flattened: stride j of KV head (b, g)
  const int c8 = static_cast<int>(gid % CH);
  if (gid >= static_cast<int64_t>(rows) * CH) return;
  const int bg = row / Ns;
  const int j = row - bg * Ns;
  const int n = min(S, L - j * S);  // keys in this stride
  const uint16_t* src = k + (static_cast<int64_t>(bg) * L + static_cast<int64_t>(j) * S) * D + c8 * 8;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  int t = 0;
  for (; t + 4 <= n; t += 4) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(t + u) * D);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += static_cast<double>(lo_bf16(w[u][e]));
        acc[2 * e + 1] += static_cast<double>(hi_bf16(w[u][e]));
      }
    }
  }
  for (; t < n; ++t) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(t) * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += static_cast<double>(lo_bf16(w[e]));
      acc[2 * e + 1] += static_cast<double>(hi_bf16(w[e]));
    }
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = f64_to_f32_round_odd(acc[2 * e] * inv_s);
    const float hi = f64_to_f32_round_odd(acc[2 * e + 1] * inv_s);
    o[e] = pack_bf16x2(lo, hi);
  }
  *reinterpret_cast<u32x4*>(kagg + static_cast<int64_t>(row) * D + c8 * 8) = o;
}

int launch_stride_aggregate(const Shape& s, const uint16_t* k, uint16_t* kagg, void* stream) {
  const int rows = s.Bz * s.Hkv * s.Ns;  // < 2^31 (checked by rra_validate)
  const int64_t threads = static_cast<int64_t>(rows) * (s.d / 8);
  if (threads == 0) return 0;
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const double inv_s = 1.0 / static_cast<double>(s.S);  // S divides Bk in {64, 128}: a power of two
  if (s.d == 128)
    hipLaunchKernelGGL(stride_aggregate_kernel<128>, dim3(blocks), dim3(256), 0, st, k, kagg, rows, s.S, s.Ns, s.L,
                       inv_s);
  else
    hipLaunchKernelGGL(stride_aggregate_kernel<64>, dim3(blocks), dim3(256), 0, st, k, kagg, rows, s.S, s.Ns, s.L,
                       inv_s);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
