// Sustained bf16 MFMA rate and shader clock (declared in rra_probe.h).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <random>
#include <vector>

#include "rra_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;   // 4 waves: one per SIMD
constexpr int kPerCU = 2;       // two workgroups per CU -> two waves per SIMD
constexpr int kCUs = 256;

__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const bf16x8* __restrict__ a, float* __restrict__ sink,
                                                             unsigned long long* __restrict__ clk, int iters) {
  const int l = threadIdx.x & 63;
  const bf16x8 x0 = a[l], x1 = a[64 + l], x2 = a[128 + l], x3 = a[192 + l];
  floatx16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((j & 1) ? x0 : x2, (j & 2) ? x1 : x3, acc[j], 0, 0, 0);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][15];
  sink[blockIdx.x * kThreads + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int rra_probe_mfma_rate(int operands, int iters, double* tflops, double* clock_ghz) {
  if (iters <= 0 || tflops == nullptr || clock_ghz == nullptr) return static_cast<int>(hipErrorInvalidValue);
  const int blocks = kCUs * kPerCU;
  std::vector<uint16_t> host(256 * 8, 0);
  if (operands != 0) {
    std::mt19937 gen(1);
    std::normal_distribution<float> nd(0.0f, 1.0f);
    for (auto& v : host) {
      const float f = nd(gen);
      uint32_t u;
      std::memcpy(&u, &f, 4);
      v = static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // round to nearest even
    }
  }
  bf16x8* a = nullptr;
  float* sink = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  std::vector<unsigned long long> hc(2 * blocks);
  float ms = 0.0f;
  hipError_t err = hipMalloc(&a, host.size() * 2);
  if (err == hipSuccess) err = hipMalloc(&sink, sizeof(float) * blocks * kThreads);
  if (err == hipSuccess) err = hipMalloc(&clk, sizeof(unsigned long long) * 2 * blocks);
  if (err == hipSuccess) err = hipMemcpy(a, host.data(), host.size() * 2, hipMemcpyHostToDevice);
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  if (err == hipSuccess) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(kThreads), 0, 0, a, sink, clk, 200);  // warm-up
    err = hipDeviceSynchronize();
  }
  if (err == hipSuccess) err = hipEventRecord(e0, 0);
  if (err == hipSuccess) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(kThreads), 0, 0, a, sink, clk, iters);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipEventRecord(e1, 0);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  if (err == hipSuccess) err = hipMemcpy(hc.data(), clk, sizeof(unsigned long long) * 2 * blocks, hipMemcpyDeviceToHost);
  if (err == hipSuccess) {
    double cyc = 0.0, rt = 0.0;
    for (int b = 0; b < blocks; ++b) {
      cyc += static_cast<double>(hc[2 * b]);
      rt += static_cast<double>(hc[2 * b + 1]);
    }
    const double flops = static_cast<double>(blocks) * (kThreads / 64) * iters * 8 * (32.0 * 32.0 * 16.0 * 2.0);
    *tflops = flops / (ms * 1e-3) / 1e12;
    *clock_ghz = (rt > 0.0) ? cyc / (rt / 100e6) / 1e9 : 0.0;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (a) (void)hipFree(a);
  if (sink) (void)hipFree(sink);
  if (clk) (void)hipFree(clk);
  return static_cast<int>(err);
}
