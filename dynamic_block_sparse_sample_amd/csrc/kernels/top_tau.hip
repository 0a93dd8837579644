// Adaptive Top-tau block selection (RRAttention §3.3, with the last query
// block protection of §4.3; the same minimal-cumulative-set rule as
// XAttention's threshold selection).
//
// One 256-thread workgroup per row (b, h, I).  The candidates are the I+1
// causal key blocks (every key block when not causal); a row with a zero total
// (a last partial query block without a sampled query: no estimate) keeps them
// all.  The candidates' block scores are
// packed into 64-bit keys (inverted float bits << 32 | J), so one ascending
// bitonic sort in LDS orders them by (score desc, J asc).  A float64 prefix
// scan over the sorted scores finds k* = the first prefix reaching
// tau * (row total); the k* selected blocks are flagged in LDS, written as the
// mask row, and compacted in ascending J order by an exclusive scan into the
// index list.
#include <climits>

#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

constexpr int kTopThreads = 256;
constexpr int kTopWaves = kTopThreads / 64;

template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* sh, T& total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  T incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kTopWaves; ++k) {
    if (k < w) base += sh[k];
    tot += sh[k];
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

__device__ __forceinline__ int block_min_int(int v, int* sh) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int k = 1; k < kTopWaves; ++k) r = min(r, sh[k]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float key_value(uint64_t key) {
  return __uint_as_float(~static_cast<uint32_t>(key >> 32));
}

// NMAX: largest row length the LDS arrays hold (a power of two >= Nb), so rows
// of short sequences do not pay the LDS, and the occupancy, of 4096 blocks.
template <int NMAX>
__global__ __launch_bounds__(kTopThreads) void top_tau_kernel(const float* __restrict__ score,
                                                              uint8_t* __restrict__ mask,
                                                              int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ cnt, int Nb,
                                                              double tau, int protect_last, int keep_all,
                                                              int causal) {
  __shared__ uint64_t keys[NMAX];
  __shared__ int flags[NMAX];
  __shared__ double dsh[kTopWaves];
  __shared__ int ish[kTopWaves];

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int I = static_cast<int>(row % Nb);
  const int n = causal ? I + 1 : Nb;  // candidate key blocks
  const float* srow = score + row * Nb;
  uint8_t* mrow = mask + row * Nb;
  int32_t* irow = idx + row * Nb;

  if (keep_all || (protect_last && I == Nb - 1) || n == 1) {
    for (int J = tid; J < Nb; J += kTopThreads) {
      mrow[J] = J < n ? 1 : 0;
      if (J < n) irow[J] = J;
    }
    if (tid == 0) cnt[row] = n;
    return;
  }

  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  for (int J = tid; J < np2; J += kTopThreads) {
    uint64_t key = ~0ull;
    if (J < n) key = (static_cast<uint64_t>(~__float_as_uint(srow[J])) << 32) | static_cast<uint32_t>(J);
    keys[J] = key;
  }
  for (int J = tid; J < Nb; J += kTopThreads) flags[J] = 0;
  __syncthreads();

  // Bitonic sort, ascending.
  for (int kk = 2; kk <= np2; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < (np2 >> 1); t += kTopThreads) {
        const int i0 = 2 * jj * (t / jj) + (t % jj);
        const int i1 = i0 + jj;
        const uint64_t a = keys[i0];
        const uint64_t bkey = keys[i1];
        const bool up = (i0 & kk) == 0;
        if ((a > bkey) == up) {
          keys[i0] = bkey;
          keys[i1] = a;
        }
      }
      __syncthreads();
    }
  }

  // Float64 prefix sums over the sorted scores.
  const int per = (n + kTopThreads - 1) / kTopThreads;
  const int p0 = tid * per;
  double tsum = 0.0;
  for (int e = 0; e < per; ++e) {
    const int p = p0 + e;
    if (p < n) tsum += static_cast<double>(key_value(keys[p]));
  }
  double total;
  double c = block_exclusive_scan<double>(tsum, dsh, total);
  const double thr = tau * total;
  int first = INT_MAX;
  for (int e = 0; e < per; ++e) {
    const int p = p0 + e;
    if (p < n) {
      c += static_cast<double>(key_value(keys[p]));
      if (c >= thr && first == INT_MAX) first = p;
    }
  }
  const int fmin = block_min_int(first, ish);
  const int kstar = (fmin == INT_MAX || !(total > 0.0)) ? n : fmin + 1;

  for (int p = tid; p < kstar; p += kTopThreads) flags[static_cast<uint32_t>(keys[p])] = 1;
  __syncthreads();
  for (int J = tid; J < Nb; J += kTopThreads) mrow[J] = static_cast<uint8_t>(flags[J]);

  // Ascending compaction of the selected J.
  int fsum = 0;
  for (int e = 0; e < per; ++e) {
    const int J = p0 + e;
    if (J < n) fsum += flags[J];
  }
  int ftotal;
  int pos = block_exclusive_scan<int>(fsum, ish, ftotal);
  for (int e = 0; e < per; ++e) {
    const int J = p0 + e;
    if (J < n && flags[J]) irow[pos++] = J;
  }
  if (tid == 0) cnt[row] = kstar;
}

int launch_top_tau(const Shape& s, float tau, int protect_last, const float* score, uint8_t* mask, int32_t* idx,
                   int32_t* cnt, void* stream) {
  const int64_t rows = static_cast<int64_t>(s.Bz) * s.H * s.Nb;
  if (rows == 0) return 0;
  const int keep_all = tau >= 1.0f ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(rows));
  const int causal = s.causal ? 1 : 0;
  const double t = static_cast<double>(tau);
  if (s.Nb <= 256)
    hipLaunchKernelGGL(top_tau_kernel<256>, grid, dim3(kTopThreads), 0, st, score, mask, idx, cnt, s.Nb, t,
                       protect_last, keep_all, causal);
  else if (s.Nb <= 1024)
    hipLaunchKernelGGL(top_tau_kernel<1024>, grid, dim3(kTopThreads), 0, st, score, mask, idx, cnt, s.Nb, t,
                       protect_last, keep_all, causal);
  else
    hipLaunchKernelGGL(top_tau_kernel<kMaxBlocks>, grid, dim3(kTopThreads), 0, st, score, mask, idx, cnt, s.Nb, t,
                       protect_last, keep_all, causal);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
