// Block-sparse causal flash attention for prefill (RRAttention §4.1: attention
// computed only on the selected key blocks; dense FlashAttention is the same
// kernel with every causal block listed).
//
// One workgroup per (batch, query head h, query block I) with BLK/32 waves;
// wave w owns 32 queries.  For each listed key block J the workgroup stages
// K[J] row-major and V[J] transposed into LDS, then every wave computes
//   S^T = K_J Q^T          (v_mfma_f32_32x32x16_bf16, A = 32 keys, B = 32 queries)
// so each lane holds one query (lane & 31) and 16 of every 32 keys.  The
// online softmax (base 2, float32) needs only in-lane reductions plus one
// exchange with lane ^ 32.  The probabilities, rounded to bf16, are already in
// the B-operand layout of the second product
//   O^T += V_J^T P^T       (A = 32 channels x 16 keys read from the V^T tile)
// once the keys of the contraction are enumerated in the order the first
// product left them in the lanes (a permutation of the summation index).
//
// Work order: longest rows (largest I) first; when the KV groups divide
// evenly over the 8 XCDs, the workgroups of one KV group are mapped to one XCD
// (workgroup w runs on XCD w mod 8) so the heads of a group and neighbouring
// query blocks share K/V tiles in that XCD's L2.
#include <cmath>

#include "../rra_internal.h"
#include "rra_device.h"

namespace rra {

template <int D, int BLK>
struct FaCfg {
  static constexpr int NW = BLK / 32;  // waves, 32 queries each
  static constexpr int NT = NW * 64;
  static constexpr int KP = D + 8;     // K tile pitch (bf16): rows 4 banks apart
  static constexpr int VP = BLK + 4;   // V^T tile pitch (bf16): rows 2 banks apart
  static constexpr int KC = D / 16;    // MFMA k-chunks of Q K^T
  static constexpr int ST = BLK / 32;  // 32-key tiles of S^T
  static constexpr int CT = D / 32;    // 32-channel tiles of O^T
  static constexpr int LDS_BYTES = (BLK * KP + D * VP) * 2;
};

enum WorkMap : int { kMapPlain = 0, kMapXcdGroups = 1, kMapXcdSplit = 2 };

template <int D, int BLK>
__global__ __launch_bounds__((BLK / 32) * 64, 2) void flash_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, uint16_t* __restrict__ out, int H,
    int Hkv, int G, int L, int Nb, float c, int map_mode) {
  using C = FaCfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
  uint16_t* Ks = lds;                // [BLK][KP]
  uint16_t* Vt = lds + BLK * C::KP;  // [D][VP]

  // ---- work item ----
  const int nbg = static_cast<int>(gridDim.x / (static_cast<unsigned>(G) * Nb));
  int bg, hh, I;
  {
    const int w = blockIdx.x;
    if (map_mode == kMapXcdGroups) {
      const int xcd = w & 7;
      int slot = w >> 3;
      const int per = nbg >> 3;
      hh = slot % G;
      slot /= G;
      const int kq = slot % per;
      I = Nb - 1 - slot / per;
      bg = xcd + 8 * kq;
    } else if (map_mode == kMapXcdSplit) {
      const int xcd = w & 7;
      int slot = w >> 3;
      const int split = 8 / nbg;
      bg = xcd % nbg;
      const int part = xcd / nbg;
      hh = slot % G;
      slot /= G;
      I = Nb - 1 - (slot * split + part);
    } else {
      int t = w;
      hh = t % G;
      t /= G;
      bg = t % nbg;
      I = Nb - 1 - t / nbg;
    }
  }
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int h = g * G + hh;
  const int64_t row = (static_cast<int64_t>(b) * H + h) * Nb + I;

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int q_local = wv * 32 + col;  // query inside the block
  const int64_t q_tok = static_cast<int64_t>(I) * BLK + q_local;

  // Q as the B operand of S^T = K Q^T: 8 consecutive channels per lane and chunk.
  bf16x8 qb[C::KC];
  {
    const uint16_t* qrow = q + ((static_cast<int64_t>(b) * H + h) * L + q_tok) * D + half * 8;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) qb[kc] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + kc * 16));
  }

  floatx16 o[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[ct][e] = 0.0f;
  float m = -INFINITY;
  float l = 0.0f;

  const int n = (idx == nullptr) ? I + 1 : cnt[row];
  const int32_t* list = (idx == nullptr) ? nullptr : idx + row * Nb;
  const uint16_t* kbase = k + static_cast<int64_t>(bg) * L * D;
  const uint16_t* vbase = v + static_cast<int64_t>(bg) * L * D;

  for (int it = 0; it < n; ++it) {
    const int J = (list == nullptr) ? it : list[it];
    const uint16_t* kblk = kbase + static_cast<int64_t>(J) * BLK * D;
    const uint16_t* vblk = vbase + static_cast<int64_t>(J) * BLK * D;

    // ---- stage K (row-major) and V (transposed) into LDS ----
    constexpr int KITEMS = BLK * D / 8;         // 16-byte chunks of the K block
    constexpr int KPER = KITEMS / C::NT;
    constexpr int VITEMS = (BLK / 4) * (D / 8);  // 4 keys x 8 channels each
    constexpr int VPER = VITEMS / C::NT;
    u32x4 kr[KPER];
    u32x4 vr[VPER][4];
#pragma unroll
    for (int e = 0; e < KPER; ++e) {
      const int item = tid + e * C::NT;
      const int rr = item / (D / 8);
      const int c8 = item % (D / 8);
      kr[e] = *reinterpret_cast<const u32x4*>(kblk + rr * D + c8 * 8);
    }
#pragma unroll
    for (int e = 0; e < VPER; ++e) {
      const int item = tid + e * C::NT;
      const int kg = (item & 15) + 16 * (item / (16 * (D / 8)));
      const int c8 = (item >> 4) % (D / 8);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vr[e][kk] = *reinterpret_cast<const u32x4*>(vblk + (4 * kg + kk) * D + c8 * 8);
    }
    __syncthreads();  // every wave is done reading the previous tiles
#pragma unroll
    for (int e = 0; e < KPER; ++e) {
      const int item = tid + e * C::NT;
      const int rr = item / (D / 8);
      const int c8 = item % (D / 8);
      *reinterpret_cast<u32x4*>(Ks + rr * C::KP + c8 * 8) = kr[e];
    }
#pragma unroll
    for (int e = 0; e < VPER; ++e) {
      const int item = tid + e * C::NT;
      const int kg = (item & 15) + 16 * (item / (16 * (D / 8)));
      const int c8 = (item >> 4) % (D / 8);
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        // channel c8*8+ch of keys 4kg..4kg+3 -> one 8-byte row segment of V^T
        const int wd = ch >> 1;
        const bool hi = ch & 1;
        uint32_t k0 = hi ? (vr[e][0][wd] >> 16) : (vr[e][0][wd] & 0xffffu);
        uint32_t k1 = hi ? (vr[e][1][wd] >> 16) : (vr[e][1][wd] & 0xffffu);
        uint32_t k2 = hi ? (vr[e][2][wd] >> 16) : (vr[e][2][wd] & 0xffffu);
        uint32_t k3 = hi ? (vr[e][3][wd] >> 16) : (vr[e][3][wd] & 0xffffu);
        u32x2 pk;
        pk[0] = k0 | (k1 << 16);
        pk[1] = k2 | (k3 << 16);
        *reinterpret_cast<u32x2*>(Vt + (c8 * 8 + ch) * C::VP + 4 * kg) = pk;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T ----
    floatx16 s[C::ST];
#pragma unroll
    for (int t = 0; t < C::ST; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[t][e] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(Ks + (32 * t + col) * C::KP + kc * 16 + half * 8);
        s[t] = mfma32x32x16(as_bf16x8(a), qb[kc], s[t]);
      }
    }

    // ---- online softmax (base 2) ----
    const bool diag = (J == I);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < C::ST; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[t][e] * c;
        if (diag) {
          const int key_local = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
          if (key_local > q_local) x = -INFINITY;
        }
        s[t][e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[ct][e] *= alpha;
    m = m_new;

    u32x4 pb[C::ST][2];
#pragma unroll
    for (int t = 0; t < C::ST; ++t) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(s[t][8 * u + 2 * e] - m_new);
          const float p1 = fast_exp2(s[t][8 * u + 2 * e + 1] - m_new);
          l += p0 + p1;
          pb[t][u][e] = pack_bf16x2(p0, p1);
        }
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const uint16_t* vrow = Vt + (32 * ct + col) * C::VP + 4 * half;
#pragma unroll
      for (int t = 0; t < C::ST; ++t) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 32 * t + 16 * u);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 32 * t + 16 * u + 8);
          u32x4 a;
          a[0] = lo[0];
          a[1] = lo[1];
          a[2] = hi[0];
          a[3] = hi[1];
          o[ct] = mfma32x32x16(as_bf16x8(a), as_bf16x8(pb[t][u]), o[ct]);
        }
      }
    }
  }

  // ---- normalise and store: lane holds 4 consecutive channels per group ----
  l += shfl_xor_f(l, 32);
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  uint16_t* orow = out + ((static_cast<int64_t>(b) * H + h) * L + q_tok) * D;
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 w;
      w[0] = pack_bf16x2(o[ct][4 * g4 + 0] * inv, o[ct][4 * g4 + 1] * inv);
      w[1] = pack_bf16x2(o[ct][4 * g4 + 2] * inv, o[ct][4 * g4 + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + 32 * ct + 8 * g4 + 4 * half) = w;
    }
  }
}

static int work_map_mode(const Shape& s) {
  const int nbg = s.Bz * s.Hkv;
  if (nbg % 8 == 0) return kMapXcdGroups;
  if (8 % nbg == 0 && s.Nb % (8 / nbg) == 0) return kMapXcdSplit;
  return kMapPlain;
}

template <int D, int BLK>
static void launch_fa(const Shape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                      const int32_t* cnt, uint16_t* out, hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(s.Bz) * s.H * s.Nb;
  hipLaunchKernelGGL((flash_attn_kernel<D, BLK>), dim3(static_cast<unsigned>(blocks)), dim3(FaCfg<D, BLK>::NT), 0,
                     st, q, k, v, idx, cnt, out, s.H, s.Hkv, s.G, s.L, s.Nb, s.scale * kLog2e, work_map_mode(s));
}

int launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                      const int32_t* cnt, uint16_t* out, void* stream) {
  if (static_cast<int64_t>(s.Bz) * s.Nb == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.d == 128 && s.Bk == 128)
    launch_fa<128, 128>(s, q, k, v, idx, cnt, out, st);
  else if (s.d == 128 && s.Bk == 64)
    launch_fa<128, 64>(s, q, k, v, idx, cnt, out, st);
  else if (s.d == 64 && s.Bk == 128)
    launch_fa<64, 128>(s, q, k, v, idx, cnt, out, st);
  else
    launch_fa<64, 64>(s, q, k, v, idx, cnt, out, st);
  return static_cast<int>(hipGetLastError());
}

}  // namespace rra
