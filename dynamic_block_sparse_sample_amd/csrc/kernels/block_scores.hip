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
// Two passes over the visible strides j <= i: pass 1 finds a reference max
// per row (its first tile's max) and the softmax denominator against it
// (base 2; the exact running max only if a denominator leaves [0, 2^100]),
// pass 2 recomputes the scores, normalises them (1/z and 1/r enter the
// exponent as log2(z r)) and sums them into block cells
//   score[b,h,I,J] = (1/r) sum_{i in I} sum_{j in J, j <= i} p[i,j]
// with in-lane adds, one permlane32 exchange per two blocks (each lane half
// then finishes a different block) and DPP sums over the r queries of a head.
// Kagg tiles (32 aggregated keys) are copied once per workgroup straight from
// global memory into LDS (global_load_lds_dwordx4), each row's 16-byte chunks
// XOR-swizzled so the A-operand reads of 32 rows are free of bank conflicts,
// in chunks of two tiles over four buffers (one barrier per chunk; a chunk's
// copies have a whole iteration to land): the four waves share every tile, a
// quarter of the L2 traffic of one wave per query block (which bound this
// kernel).
#include <climits>
#include <cmath>

#include "../rra_internal.h"
#include "lds_copy.h"
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
  constexpr int ROWB = D * 2;                    // bytes per aggregated-key row
  constexpr int RC = D / 8;                      // 16-byte chunks per row
  constexpr int TILEB = 32 * ROWB;               // bytes of one 32-row tile
  constexpr int ROWS_PER_INST = 64 / RC;         // rows per copy instruction (1 KB)
  constexpr int IPW = TILEB / 1024 / kBsWaves;   // copy instructions per wave and tile
  static_assert(TILEB % (1024 * kBsWaves) == 0, "copy split");
  // Four tile buffers (two chunks of two).
  __shared__ __attribute__((aligned(1024))) uint8_t kt[4][TILEB];
  __shared__ int s_redo;

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

  // Per-lane byte offsets that stay fixed for the whole kernel, kept in
  // registers (the empty asm makes them opaque, so the compiler does not
  // recompute them for every tile): fa[kc], the A-operand chunk of row col
  // inside a tile buffer (the buffer itself is an immediate offset), and
  // vo[i], the source of copy instruction i relative to the tile's first row.
  // A tile buffer holds row r's chunk slot s at position s ^ swz(r), which
  // keeps the A-operand reads of 32 rows free of bank conflicts.
  uint32_t fa[KC];
  {
    const int sw = swz(col) & (RC - 1);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      fa[kc] = col * ROWB + (((2 * kc + half) ^ sw) * 16);
      asm volatile("" : "+v"(fa[kc]));
    }
  }
  int vr[IPW], vo[IPW];  // row inside the tile, source offset
  static_for<IPW>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    vr[i] = (wv * IPW + i) * ROWS_PER_INST + lane / RC;
    vo[i] = vr[i] * ROWB + (((lane % RC) ^ (swz(vr[i]) & (RC - 1))) * 16);
    asm volatile("" : "+v"(vo[i]));
  });

  // Tile jt = aggregated keys jt*32 .. jt*32+31 (rows past Ns repeat row Ns-1),
  // copied straight from global memory into LDS buffer BUF: IPW 1 KB copy
  // instructions per wave, lane -> (row, chunk slot).
  const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(kbase);
  auto copy_tile = [&](int jt, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const uint32_t l0 = lds_addr(kt[BUF]) + wv * IPW * 1024;
    const uint8_t* gt = kbytes + static_cast<int64_t>(jt) * 32 * ROWB;
    if (jt * 32 + 32 <= Ns) {
      static_for<IPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        copy16_to_lds<i * 1024>(gt, vo[i], l0);
      });
    } else {
      static_for<IPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int over = max(0, jt * 32 + vr[i] - (Ns - 1));
        copy16_to_lds<i * 1024>(gt, vo[i] - over * ROWB, l0);
      });
    }
  };
  auto frag = [&](auto bufc, u32x4 (&a)[KC]) {
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) a[kc] = *reinterpret_cast<const u32x4*>(&kt[BUF][fa[kc]]);
  };
  // Runs f(jt, S^T tile) over the wave's tiles, software-pipelined: the MFMAs
  // of tile jt+1 are issued before f works on tile jt, so the MFMA unit and
  // the VALU overlap inside the wave.  Tiles are staged in chunks of two
  // (chunk c = tiles 2c, 2c+1 in LDS set c & 1, buffers 2(c & 1) and
  // 2(c & 1) + 1) with one barrier per chunk, placed between the chunk's two
  // tiles: step c issues the MFMAs of tile 2c+1 and works on tile 2c, waits
  // for its copies of chunk c+1 and at the barrier (after which every wave is
  // done with chunk c and chunk c+1 is in LDS), starts the copies of chunk
  // c+2 into chunk c's set, then issues the MFMAs of tile 2c+2 and works on
  // tile 2c+1.  A chunk's copies so have a whole step to land.  Steps come in
  // pairs (sets 0 and 1), so every buffer index is a constant.  Every wave
  // takes part in the copies and the barriers of all ntile_wg tiles.
  auto over_tiles = [&](auto&& f) {
    const int nchunk = (ntile_wg + 1) / 2;
    auto copy_chunk = [&](int c, auto setc) {
      constexpr int SET = decltype(setc)::value;
      if (2 * c < ntile_wg) copy_tile(2 * c, std::integral_constant<int, 2 * SET>{});
      if (2 * c + 1 < ntile_wg) copy_tile(2 * c + 1, std::integral_constant<int, 2 * SET + 1>{});
    };
    copy_chunk(0, std::integral_constant<int, 0>{});
    wait_vmcnt<0>();
    __syncthreads();  // chunk 0 in LDS
    if (nchunk > 1) copy_chunk(1, std::integral_constant<int, 1>{});
    floatx16 acc_a, acc_b;
    if (ntile > 0) {
      u32x4 a[KC];
      frag(std::integral_constant<int, 0>{}, a);
      acc_a = tile_mma<D>(a, qb);
    }
    auto step = [&](int c, auto setc) {
      constexpr int SET = decltype(setc)::value;
      const int t0 = 2 * c, t1 = 2 * c + 1, t2 = 2 * c + 2;
      if (t1 < ntile) {
        u32x4 a[KC];
        frag(std::integral_constant<int, 2 * SET + 1>{}, a);
        acc_b = tile_mma<D>(a, qb);
      }
      if (t0 < ntile) f(t0, acc_a);
      wait_vmcnt<0>();
      __syncthreads();
      if (c + 2 < nchunk) copy_chunk(c + 2, setc);
      if (t2 < ntile) {
        u32x4 a[KC];
        frag(std::integral_constant<int, 2 * (SET ^ 1)>{}, a);
        acc_a = tile_mma<D>(a, qb);
      }
      if (t1 < ntile) f(t1, acc_b);
    };
    for (int c = 0; c < nchunk; c += 2) {
      step(c, std::integral_constant<int, 0>{});
      if (c + 1 < nchunk) step(c + 1, std::integral_constant<int, 1>{});
    }
    __syncthreads();  // every wave is done with both sets before they are restaged
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
  // Each row's reference max is the max over its first tile, which holds
  // stride 0 (always visible), and serves the whole row, so the later tiles
  // need no max and the denominator is never rescaled.  Later scores may lie
  // above it; if some row's denominator ends outside [0, 2^100] (a score far
  // above the first tile's), the workgroup runs pass 1 again with the exact
  // running max.  Either way pass 2 normalises with the (m, z) pass 1 left.
  float m = -INFINITY, z = 0.0f;
  auto pass1_ref = [&](int jt, const floatx16& acc) {
    if (jt * 32 + 31 <= jlim) {
      if (jt == 0) {
        float tm = acc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) tm = fmaxf(tm, acc[v]);
        m = tm * c;
      }
      float zz = z;
#pragma unroll
      for (int v = 0; v < 16; ++v) zz += fast_exp2(fmaf(acc[v], c, -m));
      z = zz;
    } else {
      float x[16];
      masked(jt, acc, x);
      if (jt == 0) {
        float tm = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) tm = fmaxf(tm, x[v]);
        m = (tm > -INFINITY) ? tm : 0.0f;  // a lane without a sampled query: any finite value
      }
      float zz = z;
#pragma unroll
      for (int v = 0; v < 16; ++v) zz += (x[v] > -INFINITY) ? fast_exp2(x[v] - m) : 0.0f;
      z = zz;
    }
  };
  auto pass1_exact = [&](int jt, const floatx16& acc) {
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
  if (tid == 0) s_redo = 0;  // read only after the barriers of pass 1
  over_tiles(pass1_ref);
  if (has_q && !(z <= 0x1p100f)) s_redo = 1;
  __syncthreads();
  if (s_redo) {
    m = -INFINITY;
    z = 0.0f;
    over_tiles(pass1_exact);
  }
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
  // Pass 2 takes exp2(x - mz) with mz = m + log2(z r_I), which is already the
  // probability divided by the r_I sampled queries of the block; lanes
  // without a sampled query use mz = +inf, so theirs are 0.  (A block without
  // any sampled query so gets a zero row.)
  const float mz = has_q ? m + __builtin_amdgcn_logf(z * static_cast<float>(r_I)) : INFINITY;
  float* srow_base = score + (static_cast<int64_t>(b) * H * Nb + I) * Nb;  // + h * Nb * Nb + J

  const int jlast = causal ? I : Nb - 1;  // last key block of the row

  // ---- pass 2: probabilities pooled into block cells ----
  auto pass2 = [&](int jt, const floatx16& acc) {
    float e[16];  // probabilities / r_I
    if (jt * 32 + 31 <= jlim) {
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(acc[v], c, -mz));
    } else {
      float x[16];
      masked(jt, acc, x);
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = (x[v] > -INFINITY) ? fast_exp2(x[v] - mz) : 0.0f;
    }
    if constexpr (R >= 8) {
      // A block spans R >= 8 strides: groups of 4 values (v >> 2) in both lane halves.
      constexpr int NJ = 32 / R;
      float part[NJ];
#pragma unroll
      for (int u = 0; u < NJ; ++u) part[u] = e[(u * R) / 2];  // first value of block u in this lane
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (v != ((8 * (v >> 2)) / R) * R / 2) part[(8 * (v >> 2)) / R] += e[v];
      if constexpr (NJ >= 2) {
        // Blocks u and u+1 in one exchange: afterwards lanes 0-31 hold block
        // u's sum over both halves, lanes 32-63 block u+1's.
#pragma unroll
        for (int u = 0; u < NJ; u += 2) {
          const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[u]), __float_as_uint(part[u + 1]),
                                                          false, false);
          part[u / 2] = group_sum<R>(__uint_as_float(w[0]) + __uint_as_float(w[1]));
        }
        if (valid && (col % R) == 0) {
#pragma unroll
          for (int u = 0; u < NJ; u += 2) {
            const int J = jt * NJ + u + half;
            if (J <= jlast) srow_base[static_cast<int64_t>(h) * Nb * Nb + J] = part[u / 2];
          }
        }
      } else {
        part[0] = group_sum<R>(sum_halves(part[0]));
        if (valid && half == 0 && (col % R) == 0) {
          const int J = jt;
          if (J <= jlast) srow_base[static_cast<int64_t>(h) * Nb * Nb + J] = part[0];
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
      for (int u = 0; u < NJL; ++u) part[u] = group_sum<R>(part[u]);
      if (valid && (col % R) == 0) {
#pragma unroll
        for (int u = 0; u < NJL; ++u) {
          const int so = 8 * (u / PER) + 4 * half + R * (u % PER);  // first stride of the block in the tile
          const int J = jt * (32 / R) + so / R;
          if (J <= jlast) srow_base[static_cast<int64_t>(h) * Nb * Nb + J] = part[u];
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
