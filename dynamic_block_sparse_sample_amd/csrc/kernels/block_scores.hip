// Round-robin sampled stride scores, stride softmax and block pooling
// (RRAttention §3.1 query sampling with head round-robin, §3.2 stride-level
// importance estimation, §2.2 query independence).
//
// One workgroup of four waves per (batch, KV group g, four consecutive query
// blocks, row tile); wave w takes query block I0 - w.  A row tile holds 32
// sampled queries: strides i of block I for the G query heads of group g,
// taken at positions P(i,h) = i*S + o(h), o(h) = (rr_step * h + rr_shift) mod S
// (head round-robin: h mod S; the layer / hybrid / fixed variants of the
// §4.3 ablation change only o).  The wave computes the
// transposed score tile S^T = Kagg_tile x Q_sampled^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 aggregated keys, B = 32 sampled queries),
// so every lane owns one sampled query (lane & 31) and 16 of the 32 strides of
// a tile; the other 16 live in lane ^ 32.  Row statistics (max, sum) are then
// per-lane, with one cross-half exchange at the end.
//
// Ragged lengths: a last partial stride may hold no sampled query for a head
// (its lane contributes nothing) and a last partial block averages over the
// sampled queries it holds (a zero row when it holds none).  Without
// causality every stride and key block is visible.
//
// Two passes over the visible strides j <= i: pass 1 finds the row max and
// the softmax denominator (online, base-2), pass 2 recomputes the scores,
// normalises them and sums them into block cells
//   score[b,h,I,J] = (1/r) sum_{i in I} sum_{j in J, j <= i} p[i,j]
// with in-lane adds plus DPP / permlane sums over the r queries of a head.
// Kagg tiles (32 aggregated keys) are staged once per workgroup in LDS, rows
// padded by 16 bytes so the A-operand reads of 32 rows are free of bank
// conflicts, double-buffered with the next tile's loads in registers: the
// four waves share every tile, a quarter of the L2 traffic of one wave per
// query block (which bound this kernel).
#include <climits>
#include <cmath>

#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

template <int D>
__device__ __forceinline__ floatx16 tile_mma(const u32x4 (&a)[D / 16], const bf16x8 (&qb)[D / 16]) {
  floatx16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) acc = mfma32x32x16(as_bf16x8(a[kc]), qb[kc], acc);
  return acc;
}

constexpr int kBsWaves = 4;  // query blocks (waves) per workgroup

template <int D, int R>
__global__ __launch_bounds__(kBsWaves * 64) void block_scores_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kagg,
                                                          float* __restrict__ score, int H, int Hkv,
                                                          int G, int L, int S, int Ns, int Nb, int n_rt,
                                                          int nbg, float c, int rr_step, int rr_shift,
                                                          int causal) {
  constexpr int KC = D / 16;
  constexpr int PITCH = D * 2 + 16;      // LDS bytes per aggregated-key row
  constexpr int RC = D / 8;              // 16-byte chunks per row
  constexpr int CPT = 32 * RC / (kBsWaves * 64);  // chunks each thread stages per tile
  static_assert(32 * RC % (kBsWaves * 64) == 0, "staging split");
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][32 * PITCH];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  int wg = blockIdx.x;
  const int rt = wg % n_rt;
  wg /= n_rt;
  const int bg = wg % nbg;                        // b * Hkv + g
  const int I0 = Nb - 1 - (wg / nbg) * kBsWaves;  // longest rows first
  const int I = I0 - wv;                          // this wave's query block (< 0: idle)
  const bool active = I >= 0;
  const int b = bg / Hkv;
  const int g = bg % Hkv;

  const int rho = rt * 32 + col;    // sampled-query slot inside the group
  const bool valid = active && rho < G * R;
  const int hh = valid ? rho / R : 0;
  const int ii = rho % R;
  const int h = g * G + hh;
  const int i = I * R + ii;         // sampled stride
  const int off = (rr_step * h + rr_shift) % S;
  const int64_t pos = static_cast<int64_t>(i) * S + off;
  // A last partial stride may hold no sampled query for this head (pos >= L).
  const bool has_q = valid && pos < L;
  // Sampled queries of block I for this head: r_I = R for a whole block, fewer
  // (possibly 0) in a last partial block; the block row is their mean.
  const int n_sampled = (L > off) ? (L - off + S - 1) / S : 0;
  const int r_I = min(R, max(0, n_sampled - I * R));

  bf16x8 qb[KC];
  {
    const uint16_t* qrow = q + ((static_cast<int64_t>(b) * H + h) * L + pos) * D + half * 8;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (has_q) w = *reinterpret_cast<const u32x4*>(qrow + kc * 16);
      qb[kc] = as_bf16x8(w);
    }
  }
  const uint16_t* kbase = kagg + static_cast<int64_t>(bg) * Ns * D;
  const int nvis = causal ? (I + 1) * R : Nb * R;  // strides of the candidate blocks
  const int ntile = active ? (nvis + 31) / 32 : 0;
  const int ntile_wg = ((causal ? (I0 + 1) * R : Nb * R) + 31) / 32;  // wave 0's, the most
  const int jmax = has_q ? (causal ? i : Ns - 1) : -1;  // visible strides: j <= i (all when not causal)
  // Tiles wholly at or below the smallest visible stride of the wave need no
  // mask (lanes without a query hold Q = 0, so their scores are 0 and finite).
  int jlim = has_q ? jmax : INT_MAX;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) jlim = min(jlim, __shfl_xor(jlim, o, 64));
  jlim = __builtin_amdgcn_readfirstlane(jlim);

  // Tile jt = aggregated keys jt*32 .. jt*32+31 (rows past Ns repeat row Ns-1).
  auto load_regs = [&](int jt, u32x4 (&r)[CPT]) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int ch = tid + e * kBsWaves * 64;
      const int64_t jrow = min(jt * 32 + ch / RC, Ns - 1);
      r[e] = *reinterpret_cast<const u32x4*>(kbase + jrow * D + (ch % RC) * 8);
    }
  };
  auto store_lds = [&](int buf, const u32x4 (&r)[CPT]) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int ch = tid + e * kBsWaves * 64;
      *reinterpret_cast<u32x4*>(&kt[buf][(ch / RC) * PITCH + (ch % RC) * 16]) = r[e];
    }
  };
  auto frag = [&](int buf, u32x4 (&a)[KC]) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) a[kc] = *reinterpret_cast<const u32x4*>(&kt[buf][col * PITCH + (2 * kc + half) * 16]);
  };
  // Runs f(jt, S^T tile) over the wave's tiles, software-pipelined: the MFMAs
  // of tile jt+1 are issued before f works on tile jt, so the MFMA unit and
  // the VALU overlap inside the wave.  Every wave takes part in the staging
  // and the barriers of all ntile_wg tiles.  Tiles jt and jt+1 sit in the two
  // LDS buffers during step jt; tile jt+2 replaces tile jt at the end of the
  // step, after the barrier that followed every wave's reads of tile jt.
  auto over_tiles = [&](auto&& f) {
    u32x4 r[CPT];
    load_regs(0, r);
    store_lds(0, r);
    if (ntile_wg > 1) {
      load_regs(1, r);
      store_lds(1, r);
    }
    __syncthreads();
    floatx16 acc_cur, acc_next;
    if (ntile > 0) {
      u32x4 a[KC];
      frag(0, a);
      acc_cur = tile_mma<D>(a, qb);
    }
    __syncthreads();  // every wave has read tile 0 before step 0 refills its buffer
    for (int jt = 0; jt < ntile_wg; ++jt) {
      const int buf = jt & 1;
      const bool refill = jt + 2 < ntile_wg;
      if (refill) load_regs(jt + 2, r);
      if (jt + 1 < ntile) {
        u32x4 a[KC];
        frag(buf ^ 1, a);
        acc_next = tile_mma<D>(a, qb);
      }
      if (jt < ntile) f(jt, acc_cur);
      if (refill) store_lds(buf, r);
      __syncthreads();
      acc_cur = acc_next;
    }
  };
  // Masked base-2 logits of tile jt (only the tiles that reach past jlim).
  auto masked = [&](int jt, const floatx16& acc, float (&x)[16]) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = jt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      x[v] = (j <= jmax) ? acc[v] * c : -INFINITY;
    }
  };

  // ---- pass 1: row max and denominator (base-2 logits) ----
  float m = -INFINITY, z = 0.0f;
  auto pass1 = [&](int jt, const floatx16& acc) {
    if (jt * 32 + 31 <= jlim) {
      float tm = acc[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) tm = fmaxf(tm, acc[v]);
      const float mn = fmaxf(m, tm * c);
      float zz = z * fast_exp2(m - mn);
#pragma unroll
      for (int v = 0; v < 16; ++v) zz += fast_exp2(fmaf(acc[v], c, -mn));
      z = zz;
      m = mn;
    } else {
      float x[16];
      masked(jt, acc, x);
      float tm = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) tm = fmaxf(tm, x[v]);
      if (tm > -INFINITY) {
        const float mn = fmaxf(m, tm);
        float zz = z * fast_exp2(m - mn);
#pragma unroll
        for (int v = 0; v < 16; ++v) zz += fast_exp2(x[v] - mn);
        z = zz;
        m = mn;
      }
    }
  };
  over_tiles(pass1);
  {
    const float mo = shfl_xor_f(m, 32);
    const float zo = shfl_xor_f(z, 32);
    const float mm = fmaxf(m, mo);
    float zt = 0.0f;
    if (m > -INFINITY) zt += z * fast_exp2(m - mm);
    if (mo > -INFINITY) zt += zo * fast_exp2(mo - mm);
    m = mm;
    z = zt;
  }
  const float invz = has_q ? 1.0f / z : 0.0f;
  const float inv_r = (r_I > 0) ? 1.0f / static_cast<float>(r_I) : 0.0f;  // no sampled query: zero row
  float* srow_base = score + (static_cast<int64_t>(b) * H * Nb + I) * Nb;  // + h * Nb * Nb + J

  const int jlast = causal ? I : Nb - 1;  // last key block of the row

  // ---- pass 2: probabilities pooled into block cells ----
  auto pass2 = [&](int jt, const floatx16& acc) {
    float e[16];  // unnormalised probabilities; 1/z is applied to the in-lane sums
    if (jt * 32 + 31 <= jlim) {
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(acc[v], c, -m));
    } else {
      float x[16];
      masked(jt, acc, x);
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = (x[v] > -INFINITY) ? fast_exp2(x[v] - m) : 0.0f;
    }
    if constexpr (R >= 8) {
      // A block spans R >= 8 strides: groups of 4 values (v >> 2) in both lane halves.
      constexpr int NJ = 32 / R;
      float part[NJ];
#pragma unroll
      for (int u = 0; u < NJ; ++u) part[u] = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) part[(8 * (v >> 2)) / R] += e[v];
#pragma unroll
      for (int u = 0; u < NJ; ++u) part[u] = group_sum<R>(sum_halves(part[u] * invz));
      if (valid && half == 0 && (col % R) == 0) {
#pragma unroll
        for (int u = 0; u < NJ; ++u) {
          const int J = jt * NJ + u;
          if (J <= jlast) srow_base[static_cast<int64_t>(h) * Nb * Nb + J] = part[u] * inv_r;
        }
      }
    } else {
      // A block spans R <= 4 strides: each lane half holds whole blocks.
      constexpr int PER = 4 / R;   // blocks per 4-value group
      constexpr int NJL = 16 / R;  // blocks per lane
      float part[NJL];
#pragma unroll
      for (int u = 0; u < NJL; ++u) part[u] = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) part[(v >> 2) * PER + (v & 3) / R] += e[v];
#pragma unroll
      for (int u = 0; u < NJL; ++u) part[u] = group_sum<R>(part[u] * invz);
      if (valid && (col % R) == 0) {
#pragma unroll
        for (int u = 0; u < NJL; ++u) {
          const int so = 8 * (u / PER) + 4 * half + R * (u % PER);  // first stride of the block in the tile
          const int J = jt * (32 / R) + so / R;
          if (J <= jlast) srow_base[static_cast<int64_t>(h) * Nb * Nb + J] = part[u] * inv_r;
        }
      }
    }
  };
  over_tiles(pass2);

  // ---- zeros above the diagonal for the heads of this row tile ----
  if (!causal || !active) return;
  constexpr int HPT = 32 / R;  // heads per row tile
  for (int t = 0; t < HPT; ++t) {
    const int hz = rt * HPT + t;
    if (hz >= G) break;
    float* zrow = srow_base + static_cast<int64_t>(g * G + hz) * Nb * Nb;
    for (int J = I + 1 + lane; J < Nb; J += 64) zrow[J] = 0.0f;
  }
}

template <int D, int R>
static void launch_bs(const Shape& s, const uint16_t* q, const uint16_t* kagg, float* score, hipStream_t st) {
  const int n_rt = (s.G * R + 31) / 32;
  const int nbg = s.Bz * s.Hkv;
  const int64_t blocks = static_cast<int64_t>(n_rt) * nbg * ((s.Nb + kBsWaves - 1) / kBsWaves);
  const float c = s.scale * kLog2e;
  hipLaunchKernelGGL((block_scores_kernel<D, R>), dim3(static_cast<unsigned>(blocks)), dim3(kBsWaves * 64), 0, st,
                     q, kagg,
                     score, s.H, s.Hkv, s.G, s.L, s.S, s.Ns, s.Nb, n_rt, nbg, c, s.rr_step,
                     s.rr_shift, s.causal ? 1 : 0);
}

template <int D>
static void launch_bs_d(const Shape& s, const uint16_t* q, const uint16_t* kagg, float* score, hipStream_t st) {
  switch (s.r) {
    case 1: launch_bs<D, 1>(s, q, kagg, score, st); break;
    case 2: launch_bs<D, 2>(s, q, kagg, score, st); break;
    case 4: launch_bs<D, 4>(s, q, kagg, score, st); break;
    case 8: launch_bs<D, 8>(s, q, kagg, score, st); break;
    case 16: launch_bs<D, 16>(s, q, kagg, score, st); break;
    default: launch_bs<D, 32>(s, q, kagg, score, st); break;
  }
}

int launch_block_scores(const Shape& s, const uint16_t* q, const uint16_t* kagg, float* score, void* stream) {
  if (static_cast<int64_t>(s.Bz) * s.Nb == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.d == 128)
    launch_bs_d<128>(s, q, kagg, score, st);
  else
    launch_bs_d<64>(s, q, kagg, score, st);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
