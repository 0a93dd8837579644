// XAttention's antidiagonal block scores, kept in the library as the
// comparison estimator for pattern-search time (XAttention summary and key
// points; RRAttention §2.2 and §4.2 compare against it).
//
// Inside each S x S cell (query stride i, key stride j) of the token score
// matrix the lower-left to upper-right antidiagonal is summed:
//   a[i,j] = (sm_scale / S) * sum_o q[iS + S-1-o] . k[jS + o],
// one dot product of length S*d between the stride's queries in reverse order
// and its keys in order.  Then, as for the round-robin scores: softmax per
// query stride over j <= i, pooled into blocks with 1/r (r = Bk / S).
//
// One workgroup of 4 waves per (batch, KV group g, query block I, row tile of
// 32 query strides: strides i of block I for the G heads of group g), the same
// row tiles as the round-robin kernel.  Holding the reversed queries of the
// whole S*d contraction would take S*d/4 VGPRs per lane, so the contraction is
// split by offset o over the waves: wave w keeps the queries of offsets
// [w*S/4, (w+1)*S/4) in registers as the B operand and multiplies them with
// the matching key rows (A operand, 16 bytes per lane straight from L2) into
// a partial S^T tile.  The four partial tiles are summed through LDS (double
// buffered, one barrier per tile); afterwards wave w owns key strides
// 8w .. 8w+7 of every 32-stride tile, so the softmax statistics are merged
// over the waves once, and with r >= 8 a wave's 8 strides lie in one key
// block, pooled in registers and over the waves through LDS.
#include <cmath>

#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

template <int D, int R, int OPW>
__global__ __launch_bounds__(256, 2) void xattn_scores_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              float* __restrict__ score, int H, int Hkv, int G,
                                                              int L, int Ns, int Nb, int n_rt, int nbg, float c) {
  constexpr int KC = D / 16;
  constexpr int S = 4 * OPW;
  constexpr int HPT = 32 / R;  // heads per row tile
  constexpr int NU = 32 / R;   // key blocks per 32-stride tile
  static_assert(R >= 8 && R <= 32, "a wave's 8 strides must lie in one key block");
  __shared__ float part[2][4][16][64];
  __shared__ float stat[2][4][64];
  __shared__ float pool[2][4][HPT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  int wg = blockIdx.x;
  const int rt = wg % n_rt;
  wg /= n_rt;
  const int bg = wg % nbg;
  const int I = Nb - 1 - wg / nbg;  // longest rows first
  const int b = bg / Hkv;
  const int g = bg % Hkv;

  const int rho = rt * 32 + col;
  const bool valid = rho < G * R;
  const int hh = valid ? rho / R : 0;
  const int h = g * G + hh;
  const int i = I * R + rho % R;  // query stride

  // B operand: the stride's queries in reverse order, this wave's offsets.
  bf16x8 qb[OPW][KC];
#pragma unroll
  for (int oo = 0; oo < OPW; ++oo) {
    const int o = wv * OPW + oo;
    const uint16_t* qrow = q + ((static_cast<int64_t>(b) * H + h) * L + static_cast<int64_t>(i) * S + (S - 1 - o)) * D +
                           half * 8;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid) w = *reinterpret_cast<const u32x4*>(qrow + kc * 16);
      qb[oo][kc] = as_bf16x8(w);
    }
  }
  const uint16_t* kbase = k + static_cast<int64_t>(bg) * L * D + half * 8;
  const int ntile = ((I + 1) * R + 31) / 32;
  const int jmax = valid ? i : -1;

  // Partial S^T tile over this wave's offsets (A = keys jS + o, 32 strides j).
  auto tile_acc = [&](int jt) {
    floatx16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    const int64_t jrow = min(jt * 32 + col, Ns - 1);
#pragma unroll
    for (int oo = 0; oo < OPW; ++oo) {
      const uint16_t* krow = kbase + (jrow * S + wv * OPW + oo) * D;
      u32x4 a[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) a[kc] = *reinterpret_cast<const u32x4*>(krow + kc * 16);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) acc = mfma32x32x16(as_bf16x8(a[kc]), qb[oo][kc], acc);
    }
    return acc;
  };
  // Full logits of this wave's 4 values (key strides jt*32 + 8 wv + 4 half + e).
  auto reduce_tile = [&](int jt, const floatx16& acc, float (&x)[4]) {
    const int buf = jt & 1;
#pragma unroll
    for (int v = 0; v < 16; ++v) part[buf][wv][v][lane] = acc[v];
    __syncthreads();  // the other buffer is rewritten only after the next barrier
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) t += part[buf][w][4 * wv + e][lane];
      const int j = jt * 32 + 8 * wv + 4 * half + e;
      x[e] = (j <= jmax) ? t * c : -INFINITY;
    }
  };

  // ---- pass 1: row max and denominator over this wave's strides, then merged ----
  float m = -INFINITY, z = 0.0f;
  for (int jt = 0; jt < ntile; ++jt) {
    const floatx16 acc = tile_acc(jt);
    float x[4];
    reduce_tile(jt, acc, x);
    const float tm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (tm > -INFINITY) {
      const float mn = fmaxf(m, tm);
      float zz = z * fast_exp2(m - mn);
#pragma unroll
      for (int e = 0; e < 4; ++e) zz += fast_exp2(x[e] - mn);
      z = zz;
      m = mn;
    }
  }
  {
    const float mo = shfl_xor_f(m, 32);
    const float zo = shfl_xor_f(z, 32);
    const float mm = fmaxf(m, mo);
    float zt = 0.0f;
    if (m > -INFINITY) zt += z * fast_exp2(m - mm);
    if (mo > -INFINITY) zt += zo * fast_exp2(mo - mm);
    stat[0][wv][lane] = mm;
    stat[1][wv][lane] = zt;
    __syncthreads();
    float mall = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mall = fmaxf(mall, stat[0][w][lane]);
    float zall = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = stat[0][w][lane];
      if (mw > -INFINITY) zall += stat[1][w][lane] * fast_exp2(mw - mall);
    }
    m = mall;
    z = zall;
  }
  const float invz = valid ? 1.0f / z : 0.0f;
  const float inv_r = 1.0f / static_cast<float>(R);
  const int h0 = g * G + rt * HPT;  // first head of this row tile

  // ---- pass 2: probabilities pooled into block cells ----
  for (int jt = 0; jt < ntile; ++jt) {
    const floatx16 acc = tile_acc(jt);
    float x[4];
    reduce_tile(jt, acc, x);
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) t += (x[e] > -INFINITY) ? fast_exp2(x[e] - m) * invz : 0.0f;
    t += shfl_xor_f(t, 32);  // strides 8 wv + 4 .. 8 wv + 7
#pragma unroll
    for (int off = 1; off < R; off <<= 1) t += shfl_xor_f(t, off);  // the r query strides of the head
    const int buf = jt & 1;
    if (half == 0 && (col % R) == 0) pool[buf][wv][col / R] = t;
    __syncthreads();
    if (tid < NU * HPT) {
      const int u = tid / HPT;
      const int hz = tid % HPT;
      const int J = jt * NU + u;
      if (rt * HPT + hz < G && J <= I) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < R / 8; ++w) sum += pool[buf][u * (R / 8) + w][hz];
        score[((static_cast<int64_t>(b) * H + h0 + hz) * Nb + I) * Nb + J] = sum * inv_r;
      }
    }
  }

  // ---- zeros above the diagonal for the heads of this row tile ----
  for (int hz = 0; hz < HPT; ++hz) {
    if (rt * HPT + hz >= G) break;
    float* zrow = score + ((static_cast<int64_t>(b) * H + h0 + hz) * Nb + I) * Nb;
    for (int J = I + 1 + tid; J < Nb; J += 256) zrow[J] = 0.0f;
  }
}

template <int D, int R, int OPW>
static void launch_xa(const Shape& s, const uint16_t* q, const uint16_t* k, float* score, hipStream_t st) {
  const int n_rt = (s.G * R + 31) / 32;
  const int nbg = s.Bz * s.Hkv;
  const int64_t blocks = static_cast<int64_t>(n_rt) * nbg * s.Nb;
  const float c = s.scale * kLog2e / static_cast<float>(s.S);
  hipLaunchKernelGGL((xattn_scores_kernel<D, R, OPW>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, q, k,
                     score, s.H, s.Hkv, s.G, s.L, s.Ns, s.Nb, n_rt, nbg, c);
}

template <int D>
static int launch_xa_d(const Shape& s, const uint16_t* q, const uint16_t* k, float* score, hipStream_t st) {
  // (Bk, S) -> (R, S / 4): 128/16 -> (8, 4), 128/8 -> (16, 2), 128/4 -> (32, 1), 64/8 -> (8, 2), 64/4 -> (16, 1)
  if (s.r == 8 && s.S == 16) launch_xa<D, 8, 4>(s, q, k, score, st);
  else if (s.r == 16 && s.S == 8) launch_xa<D, 16, 2>(s, q, k, score, st);
  else if (s.r == 32 && s.S == 4) launch_xa<D, 32, 1>(s, q, k, score, st);
  else if (s.r == 8 && s.S == 8) launch_xa<D, 8, 2>(s, q, k, score, st);
  else if (s.r == 16 && s.S == 4) launch_xa<D, 16, 1>(s, q, k, score, st);
  else return -1;
  return 0;
}

int launch_xattn_scores(const Shape& s, const uint16_t* q, const uint16_t* k, float* score, void* stream) {
  if (static_cast<int64_t>(s.Bz) * s.Nb == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rc = (s.d == 128) ? launch_xa_d<128>(s, q, k, score, st) : launch_xa_d<64>(s, q, k, score, st);
  if (rc != 0) return rc;
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
