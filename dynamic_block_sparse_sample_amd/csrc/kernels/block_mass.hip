// Exact block masses of full causal attention: the reference against which
// the estimator's block selection is scored.
//
//   mass[b,h,I,J] = (1/Bk) * sum_{t in block I} sum_{u in block J, u <= t} p[t,u],
//   p[t,u] = softmax over u <= t of sm_scale * q_t . k_u,
//
// so every row sums to 1 and J > I is 0.  This is the estimator's block score
// with S = 1 (every query sampled, every key its own stride: RRAttention §3.2
// without the sampling and aggregation approximations), and Top-tau on it is
// the exact selection the sampled estimate stands in for (§3.3).
//
// One workgroup of BLK/32 waves per (b, h, I); wave w owns 32 queries whose Q
// stays in registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
// one query per lane, 16 of every 32 keys per lane, the other 16 in lane ^ 32).
// Key sub-tiles of 64 keys are staged in LDS (row pitch padded by 16 bytes so
// the A-operand reads of 32 consecutive rows are free of bank conflicts),
// double-buffered with the next sub-tile's global loads in registers.
// Pass 1 forms each query's row max and denominator (base 2, float32); pass 2
// recomputes the scores, normalises them and sums them per key block: in-lane,
// over the wave, then over the waves through LDS.  Ragged lengths: key rows
// past the end repeat row L-1 and are masked, queries past the end count for
// nothing, and a last partial block averages over the queries it has.
// Without causality every key inside the sequence is visible.
#include <cmath>

#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

template <int D, int BLK>
struct BmCfg {
  static constexpr int NW = BLK / 32;
  static constexpr int NT = NW * 64;
  static constexpr int KT = 64;               // keys per sub-tile
  static constexpr int SUB = BLK / KT;        // sub-tiles per key block
  static constexpr int RC = D / 8;            // 16-byte chunks per key row
  static constexpr int PITCH = D * 2 + 16;    // LDS bytes per key row
  static constexpr int CPT = KT * RC / NT;    // 16-byte chunks each thread stages per sub-tile
  static constexpr int KC = D / 16;
  static_assert(KT * RC % NT == 0, "staging split");
};

template <int D, int BLK>
__global__ __launch_bounds__((BLK / 32) * 64, 2) void block_mass_kernel(const uint16_t* __restrict__ q,
                                                                        const uint16_t* __restrict__ k,
                                                                        float* __restrict__ mass, int H, int Hkv,
                                                                        int G, int L, int Nb, float c,
                                                                        int causal) {
  using C = BmCfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][C::KT * C::PITCH];
  __shared__ float red[2][C::NW];

  // Work item: longest rows first, the heads of a KV group next to each other.
  const int nbg = static_cast<int>(gridDim.x / (static_cast<unsigned>(G) * Nb));
  int t = blockIdx.x;
  const int hh = t % G;
  t /= G;
  const int bg = t % nbg;
  const int I = Nb - 1 - t / nbg;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int h = g * G + hh;
  const int64_t row = (static_cast<int64_t>(b) * H + h) * Nb + I;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q_tok = I * BLK + wv * 32 + col;
  const bool q_in = q_tok < L;
  const int key_lim = causal ? q_tok : L - 1;  // last visible key
  const int n_q = min(BLK, L - I * BLK);       // queries in block I

  bf16x8 qb[C::KC];
  {
    const uint16_t* qrow = q + ((static_cast<int64_t>(b) * H + h) * L + (q_in ? q_tok : L - 1)) * D + half * 8;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) qb[kc] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + kc * 16));
  }
  const uint16_t* kbase = k + static_cast<int64_t>(bg) * L * D;
  const int nsub = (causal ? I + 1 : Nb) * C::SUB;

  auto load_regs = [&](int s, u32x4 (&r)[C::CPT]) {
    const int64_t key0 = static_cast<int64_t>(s) * C::KT;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      const int64_t key = min(key0 + ch / C::RC, static_cast<int64_t>(L - 1));  // rows past the end: row L-1
      r[i] = *reinterpret_cast<const u32x4*>(kbase + key * D + (ch % C::RC) * 8);
    }
  };
  auto store_lds = [&](int buf, const u32x4 (&r)[C::CPT]) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      *reinterpret_cast<u32x4*>(&kt[buf][(ch / C::RC) * C::PITCH + (ch % C::RC) * 16]) = r[i];
    }
  };
  // Base-2 logits of sub-tile s for this lane's query (keys after the query: -inf).
  auto logits = [&](int s, int buf, float (&x)[32]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      floatx16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(&kt[buf][(32 * tt + col) * C::PITCH + (2 * kc + half) * 16]);
        acc = mfma32x32x16(as_bf16x8(a), qb[kc], acc);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = s * C::KT + 32 * tt + 8 * (e >> 2) + 4 * half + (e & 3);
        x[16 * tt + e] = (key <= key_lim) ? acc[e] * c : -INFINITY;
      }
    }
  };

  // ---- pass 1: row max and denominator ----
  float m = -INFINITY, l = 0.0f;
  {
    u32x4 r[C::CPT];
    load_regs(0, r);
    store_lds(0, r);
    __syncthreads();
    for (int s = 0; s < nsub; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsub) load_regs(s + 1, r);
      float x[32];
      logits(s, buf, x);
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 32; ++e) mx = fmaxf(mx, x[e]);
      const float m_new = fmaxf(m, max_halves(mx));  // finite: key 0 is visible to every query
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) sum += fast_exp2(x[e] - m_new);
      l = l * fast_exp2(m - m_new) + sum;
      m = m_new;
      if (s + 1 < nsub) store_lds(buf ^ 1, r);  // buffer read in iteration s - 1, released by its barrier
      __syncthreads();
    }
  }
  const float inv = q_in ? 1.0f / sum_halves(l) : 0.0f;  // queries past the end count for nothing

  // ---- pass 2: normalised probabilities summed per key block ----
  float* mrow = mass + row * Nb;
  {
    u32x4 r[C::CPT];
    load_regs(0, r);
    store_lds(0, r);
    __syncthreads();
    float acc = 0.0f;
    for (int s = 0; s < nsub; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsub) load_regs(s + 1, r);
      float x[32];
      logits(s, buf, x);
#pragma unroll
      for (int e = 0; e < 32; ++e) acc += fast_exp2(x[e] - m);
      const bool block_end = (s + 1) % C::SUB == 0;
      const int J = s / C::SUB;
      if (block_end) {
        float v = acc * inv;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += shfl_xor_f(v, off);
        if (lane == 0) red[J & 1][wv] = v;
        acc = 0.0f;
      }
      if (s + 1 < nsub) store_lds(buf ^ 1, r);
      __syncthreads();
      // red[J & 1] is next written two key blocks later, after two more barriers.
      if (block_end && tid == 0) {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) tot += red[J & 1][w];
        mrow[J] = tot / static_cast<float>(n_q);
      }
    }
  }
  if (causal)
    for (int J = I + 1 + tid; J < Nb; J += C::NT) mrow[J] = 0.0f;
}

template <int D, int BLK>
static void launch_bm(const Shape& s, const uint16_t* q, const uint16_t* k, float* mass, hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(s.Bz) * s.H * s.Nb;
  hipLaunchKernelGGL((block_mass_kernel<D, BLK>), dim3(static_cast<unsigned>(blocks)), dim3(BmCfg<D, BLK>::NT), 0,
                     st, q, k, mass, s.H, s.Hkv, s.G, s.L, s.Nb, s.scale * kLog2e, s.causal ? 1 : 0);
}

int launch_block_mass(const Shape& s, const uint16_t* q, const uint16_t* k, float* mass, void* stream) {
  if (static_cast<int64_t>(s.Bz) * s.Nb == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.d == 128 && s.Bk == 128)
    launch_bm<128, 128>(s, q, k, mass, st);
  else if (s.d == 128 && s.Bk == 64)
    launch_bm<128, 64>(s, q, k, mass, st);
  else if (s.d == 64 && s.Bk == 128)
    launch_bm<64, 128>(s, q, k, mass, st);
  else
    launch_bm<64, 64>(s, q, k, mass, st);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
