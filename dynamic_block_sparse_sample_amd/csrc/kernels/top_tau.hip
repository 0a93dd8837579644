// Adaptive Top-tau block selection (RRAttention §3.3, with the last query
// block protection of §4.3; the same minimal-cumulative-set rule as
// XAttention's threshold selection).
//
// Per row (b, h, I) the candidates are the I+1 causal key blocks (every key
// block when not causal).  In the order (score desc, J asc) the selection is
// the shortest prefix whose sum reaches tau * T, T the row total; a row with
// T = 0 (a last partial query block without a sampled query: no estimate)
// keeps every candidate.
//
// No sort is needed.  One wave per row holds the row in registers (block J in
// lane J mod 64, slot J / 64; a row runs with the fewest slots, a power of
// two, that hold its candidates).  Scores are non-negative, so their float bit
// patterns order like the values; the threshold value t is found by a
// bitwise search over those 31 bits: t = the largest x with
// sum(scores >= x) >= tau * T (float32 sums, one wave reduction per bit, the
// answer then confirmed with two float64 sums, or searched again in float64).
// Every block scoring above t is then selected (their sum is below tau * T),
// and of the blocks equal to t the m lowest J, m the smallest count with
// sum(above) + m * t >= tau * T: exactly the prefix of the sorted order.
// Ranks among equal scores and the ascending compaction of the selected J
// come from per-slot ballots (a popcount of the lanes below).
#include <cmath>

#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

constexpr int kTopWaves = 4;  // rows per 256-thread workgroup

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xffffffffu), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                                     static_cast<uint32_t>(lo)));
}

// Sum over the 64 lanes, the same value in every lane: each step adds a
// lane's value and its partner's, and the partner adds the same two numbers.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppRowMirror>(v);
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const auto lo16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
  const auto hi16 =
      __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
  v = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi16[0]) << 32) | lo16[0])) +
      __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi16[1]) << 32) | lo16[1]));
  const uint64_t w = static_cast<uint64_t>(__double_as_longlong(v));
  const auto lo32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w), static_cast<uint32_t>(w), false, false);
  const auto hi32 =
      __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w >> 32), static_cast<uint32_t>(w >> 32), false, false);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi32[0]) << 32) | lo32[0])) +
         __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi32[1]) << 32) | lo32[1]));
}

// Lanes below this one among the set bits of a ballot.
__device__ __forceinline__ int lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(ballot), 0));
}

// Rows of one slot-count class: NS slots in registers (NS * 64 >= candidates;
// slots past the candidates hold zeros, which no threshold x >= 1 counts).
template <int NS>
__device__ __forceinline__ void top_tau_row(const float* __restrict__ srow, uint8_t* __restrict__ mrow,
                                            int32_t* __restrict__ irow, int32_t* __restrict__ cnt_out, int lane,
                                            int n, int Nb, double tau) {
  constexpr bool kKeepD = NS <= 16;
  uint32_t bits[NS];
  double val[kKeepD ? NS : 1];
  auto value = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (kKeepD) return val[k];
    else return static_cast<double>(__uint_as_float(bits[k]));
  };
  double total = 0.0;
  static_for<NS>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    const int J = k * 64 + lane;
    const float v = J < n ? srow[J] : 0.0f;
    bits[k] = v > 0.0f ? __float_as_uint(v) : 0u;  // zeros and non-candidates: 0
    if constexpr (kKeepD) val[k] = v > 0.0f ? static_cast<double>(v) : 0.0;
    total += value(kc);
  });
  total = wave_sum_d(total);
  if (!(total > 0.0)) {  // no estimate: every candidate (the same in every lane)
    for (int J = lane; J < Nb; J += 64) {
      mrow[J] = J < n ? 1 : 0;
      if (J < n) irow[J] = J;
    }
    if (lane == 0) *cnt_out = n;
    return;
  }

  // Threshold bits: the largest x with sum(bits >= x) >= tau * T (x >= 1,
  // since the positive scores sum to T >= tau * T).  The bitwise search runs
  // on float32 sums (cheap); its answer is then checked exactly in float64:
  // sum(>= x) >= tau * T > sum(> x) makes x the largest such value (the sum
  // only falls as x grows).  A row where float32 rounding decided a step
  // differently (a sum within ~1e-6 of tau * T) repeats the search in float64.
  const double thr = tau * total;
  auto sum_ge = [&](uint32_t cand) {
    double s = 0.0;
    static_for<NS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      s += bits[k] >= cand ? value(kc) : 0.0;
    });
    return wave_sum_d(s);
  };
  uint32_t x = 0;
  {
    const float thr32 = static_cast<float>(thr);
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = x | (1u << bit);
      float s = 0.0f;
      static_for<NS>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        s += bits[k] >= cand ? __uint_as_float(bits[k]) : 0.0f;
      });
      s = sum_halves(group_sum<32>(s));
      if (__builtin_amdgcn_readfirstlane(s >= thr32 ? 1 : 0)) x = cand;
    }
  }
  const bool exact = x >= 1 && sum_ge(x) >= thr && !(x < 0x7F800000u && sum_ge(x + 1) >= thr);
  if (!__builtin_amdgcn_readfirstlane(exact ? 1 : 0)) {
    x = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = x | (1u << bit);
      if (__builtin_amdgcn_readfirstlane(sum_ge(cand) >= thr ? 1 : 0)) x = cand;
    }
  }

  // Blocks above t, and the number of blocks equal to t.
  double above = 0.0;
  int n_eq = 0;
  static_for<NS>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    above += bits[k] > x ? value(kc) : 0.0;
    n_eq += __popcll(__ballot(bits[k] == x));
  });
  above = wave_sum_d(above);
  const double t = static_cast<double>(__uint_as_float(x));
  // m: the fewest blocks equal to t that bring the sum to tau * T (1 <= m <= n_eq).
  int m = 1;
  {
    const double need = (thr - above) / t;
    if (need > 1.0) m = need < static_cast<double>(n_eq) ? static_cast<int>(ceil(need)) : n_eq;
    while (m > 1 && above + static_cast<double>(m - 1) * t >= thr) --m;
    while (m < n_eq && above + static_cast<double>(m) * t < thr) ++m;
  }
  m = __builtin_amdgcn_readfirstlane(m);

  // Mask row, and the selected J compacted in ascending order.
  int eq_before = 0, sel_before = 0;
  static_for<NS>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    const int J = k * 64 + lane;
    const bool eq = bits[k] == x;
    const uint64_t be = __ballot(eq);
    const bool sel = bits[k] > x || (eq && eq_before + lanes_below(be) < m);
    eq_before += __popcll(be);
    if (J < Nb) mrow[J] = sel ? 1 : 0;
    const uint64_t bs = __ballot(sel);
    if (sel) irow[sel_before + lanes_below(bs)] = J;
    sel_before += __popcll(bs);
  });
  for (int J = NS * 64 + lane; J < Nb; J += 64) mrow[J] = 0;  // beyond the candidates' slots
  if (lane == 0) *cnt_out = sel_before;
}

// SLOTS: 64-block slots the largest row needs (Nb <= 64 * SLOTS).
template <int SLOTS>
__global__ __launch_bounds__(64 * kTopWaves) void top_tau_kernel(const float* __restrict__ score,
                                                                 uint8_t* __restrict__ mask,
                                                                 int32_t* __restrict__ idx,
                                                                 int32_t* __restrict__ cnt, int64_t rows, int Nb,
                                                                 double tau, int protect_last, int keep_all,
                                                                 int causal) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));  // uniform: scalar row
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTopWaves + wv;
  if (row >= rows) return;  // whole waves; no workgroup barrier below
  const int I = static_cast<int>(row % Nb);
  const int n = causal ? I + 1 : Nb;  // candidate key blocks
  const float* srow = score + row * Nb;
  uint8_t* mrow = mask + row * Nb;
  int32_t* irow = idx + row * Nb;
  int32_t* crow = cnt + row;

  if (keep_all || (protect_last && I == Nb - 1) || n == 1) {
    for (int J = lane; J < Nb; J += 64) {
      mrow[J] = J < n ? 1 : 0;
      if (J < n) irow[J] = J;
    }
    if (lane == 0) *crow = n;
    return;
  }
  const int ns = (n + 63) >> 6;  // slots holding candidates
  if (ns <= 1) top_tau_row<1>(srow, mrow, irow, crow, lane, n, Nb, tau);
  else if (SLOTS >= 2 && ns <= 2) top_tau_row<(SLOTS >= 2 ? 2 : 1)>(srow, mrow, irow, crow, lane, n, Nb, tau);
  else if (SLOTS >= 4 && ns <= 4) top_tau_row<(SLOTS >= 4 ? 4 : 1)>(srow, mrow, irow, crow, lane, n, Nb, tau);
  else if (SLOTS >= 8 && ns <= 8) top_tau_row<(SLOTS >= 8 ? 8 : 1)>(srow, mrow, irow, crow, lane, n, Nb, tau);
  else if (SLOTS >= 16 && ns <= 16) top_tau_row<(SLOTS >= 16 ? 16 : 1)>(srow, mrow, irow, crow, lane, n, Nb, tau);
  else if (SLOTS >= 32 && ns <= 32) top_tau_row<(SLOTS >= 32 ? 32 : 1)>(srow, mrow, irow, crow, lane, n, Nb, tau);
  else top_tau_row<SLOTS>(srow, mrow, irow, crow, lane, n, Nb, tau);
}

int launch_top_tau(const Shape& s, float tau, int protect_last, const float* score, uint8_t* mask, int32_t* idx,
                   int32_t* cnt, void* stream) {
  const int64_t rows = static_cast<int64_t>(s.Bz) * s.H * s.Nb;
  if (rows == 0) return 0;
  const int keep_all = tau >= 1.0f ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>((rows + kTopWaves - 1) / kTopWaves));
  const dim3 block(64 * kTopWaves);
  const int causal = s.causal ? 1 : 0;
  const double t = static_cast<double>(tau);
  if (s.Nb <= 256)
    hipLaunchKernelGGL(top_tau_kernel<4>, grid, block, 0, st, score, mask, idx, cnt, rows, s.Nb, t, protect_last,
                       keep_all, causal);
  else if (s.Nb <= 1024)
    hipLaunchKernelGGL(top_tau_kernel<16>, grid, block, 0, st, score, mask, idx, cnt, rows, s.Nb, t, protect_last,
                       keep_all, causal);
  else
    hipLaunchKernelGGL(top_tau_kernel<kMaxBlocks / 64>, grid, block, 0, st, score, mask, idx, cnt, rows, s.Nb, t,
                       protect_last, keep_all, causal);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
