// Device-side helpers shared by the gfx950 kernels.
#ifndef RRA_DEVICE_H_
#define RRA_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

namespace rra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Low / high bf16 of a packed 32-bit word, widened to float (exact).
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, in float32 (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// max(v[lane], v[lane ^ 32]) on every lane, through v_permlane32_swap (VALU, no LDS).
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// v[lane] + v[lane ^ 32] on every lane.
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v[lane] + v[lane ^ 16] on every lane (v_permlane16_swap: odd and even 16-lane rows).
__device__ __forceinline__ float sum_rows16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane permutations inside 16-lane rows (DPP controls).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15 - i
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7 - i (in each half row)

// (Every control here stays inside a 16-lane row, so bound_ctrl never applies;
// setting it lets the compiler fuse the move into the consuming add.)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of v over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32),
// in every lane of the group.  The mirrors pair lane i with its reflection, so
// after them each pair sum sits in the first half of the group and the quad
// steps finish it.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group size");
  if constexpr (N == 32) v = sum_rows16(v);
  if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  return v;
}

// f(std::integral_constant<int, 0>) ... f(std::integral_constant<int, N-1>),
// unrolled at compile time (indices stay constants, so per-index register
// arrays and immediates stay in registers and instructions).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace rra

#endif  // RRA_DEVICE_H_
