// Block-sparse flash attention for prefill (RRAttention §4.1: attention
// computed only on the selected key blocks; dense FlashAttention is the same
// kernel with every causal block listed).  Causal by default; without the
// causal mask for encoder-style use.
//
// One work item per (batch, query head h, query block I), run by a workgroup
// of BLK/32 waves (see Schedule below); wave w owns 32 queries.  Key blocks
// are consumed in 64-key sub-tiles.
//
// Data movement: K and V sub-tiles (64 keys x d, row-major) are copied from
// global memory straight into LDS with global_load_lds_dwordx4 (lane l's 16
// bytes land at LDS base + 16 l); no VGPRs are spent on staging.  K and V each
// have a ring of two LDS buffers and K runs one sub-tile ahead of V, so in
// iteration s the copies of V(s+1) and K(s+2) are in flight while the MFMA
// unit computes S(s+1) = K(s+1) Q^T and the VALU turns S(s) into
// probabilities, followed by O += V(s) P(s).  Each 256-byte key row keeps its
// sixteen 16-byte chunks XOR-swizzled by a function of the row, chosen so
// that both LDS read patterns below are free of bank conflicts with 32 or 64
// banks.
//
// Compute per sub-tile and wave:
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16, A = 32 keys (ds_read_b128 from
//                  LDS), B = 32 queries (registers).  Each lane then holds one
//                  query (lane & 31) and 16 of every 32 keys, so the online
//                  softmax (base 2, float32) is in-lane plus one exchange with
//                  lane ^ 32 (v_permlane32_swap).
//   O^T += V^T P^T A = 32 channels x 16 keys, read with ds_read_b64_tr_b16:
//                  in each 16-lane group, lane i receives element i mod 4 of
//                  the 8-byte rows addressed by lanes i/4 + 4m (m = 0..3), i.e.
//                  4 consecutive keys of one channel; B = the bf16
//                  probabilities, already in place once the contraction's keys
//                  are enumerated in the order the first product left them.
// The 16 MFMAs of S(s+1) are written in chunks, each with one pair of
// probabilities of S(s) and the LDS read of a K fragment four MFMAs ahead,
// and the compiler interleaves the whole stream (MFMA and VALU work overlap in
// one wave); the wave raises its issue priority (s_setprio) for that stream.
// The P V products that follow keep a fixed order (sched_barrier).
// Reference max: each row's max over its first sub-tile (which always holds a
// visible key) is used for the whole row, so the later sub-tiles need no row
// max and O and l are never rescaled.  Later probabilities may exceed 1;
// bf16 and float32 carry them with the same relative precision.  If some
// row's denominator ends above 2^64 (or overflows: a later logit far above the
// first sub-tile's), the item stores nothing and runs again with the exact
// running max (O and l rescaled on sub-tiles where some row's max rose).
//
// Ragged lengths (L not a multiple of the block): rows of K and V beyond the
// sequence are never read (copies of a tail sub-tile repeat row L-1, whose
// keys are masked), Q rows beyond it load row L-1 and are not stored.
// Without causality every key block is a candidate and only keys beyond the
// sequence are masked.
//
// Work order (fa_order.h): KV groups in phases small enough for the
// memory-side cache; inside a phase longest rows (largest I) first (item w
// goes to XCD w mod 8), the heads of a group adjacent so that they stream the
// same K/V through one L2, the group served by an XCD rotating every 16 slots
// so that denser groups do not leave other XCDs idle.
//
// Schedule: with a counter workspace the grid is the resident workgroups
// (occupancy x CUs, workgroup w on XCD w mod 8); each takes items w = 8k + x
// from its XCD's queue with an atomic counter and, when that queue is empty,
// from the other XCDs' queues.  The XCDs run at different clocks under the
// power limit (measured up to 5 % apart for the same work), and a static
// split leaves the fast ones idle while the slow ones finish.  Without the
// workspace every item is its own workgroup.  Each item is computed the same
// way either way, so the outputs are bitwise identical.
#include <atomic>
#include <cmath>
#include <type_traits>
#include <utility>

#include "../rra_internal.h"
#include "fa_order.h"
#include "lds_copy.h"
#include "rra_device.h"

namespace rra {

typedef short short4_t __attribute__((ext_vector_type(4)));

template <int D, int BLK>
struct FaCfg {
  static constexpr int NW = BLK / 32;          // waves, 32 queries each
  static constexpr int NT = NW * 64;
  static constexpr int KT = 64;                // keys per sub-tile
  static constexpr int SUB = BLK / KT;         // sub-tiles per key block
  static constexpr int RC = D / 8;             // 16-byte chunks per key row
  static constexpr int ROWB = D * 2;           // bytes per key row
  static constexpr int TILE = KT * ROWB;       // bytes of one K (or V) sub-tile
  static constexpr int STAGE = 2 * TILE;       // K then V
  static constexpr int NINST = KT * RC / 64;   // 1 KB copy instructions per sub-tile (each of K, V)
  static constexpr int IPW = NINST / NW;       // ... per wave
  static constexpr int ROWS_PER_INST = 64 / RC;
  static constexpr int KC = D / 16;            // MFMA k-chunks of Q K^T
  static constexpr int CT = D / 32;            // 32-channel tiles of O^T
  static_assert(NINST % NW == 0, "copy split");
};

// Workgroup barrier that does not wait for global loads in flight (the copy
// of the next sub-tile).  The only LDS writes in the loop are those copies; a
// wave's own copies of the current sub-tile are completed by wait_vmcnt before
// it arrives, so after the barrier every wave's copies have landed.  The empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier after this wave's LDS reads of a stage have completed (lgkmcnt(0),
// vmcnt untouched), so no wave refills the stage while another reads it.
__device__ __forceinline__ void lds_reads_done_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// Two workgroups per CU (64 KB of LDS each): two waves per SIMD for BLK = 128,
// one for BLK = 64 (two waves per workgroup).
template <int D, int BLK>
__global__ __launch_bounds__((BLK / 32) * 64, BLK == 128 ? 2 : 1) void flash_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, uint16_t* __restrict__ out, int H,
    int Hkv, int G, int L, int Nb, float c, int gp, int causal, int nbg, uint32_t* __restrict__ sched) {
  using C = FaCfg<D, BLK>;
  // K and V rings of two sub-tiles each (K(t) in kb[t & 1], V(t) in vb[t & 1]),
  // in distinct LDS objects so every access names its buffer statically.
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[C::TILE];

  __shared__ int s_item;
  __shared__ int s_redo;

  // ---- one work item: (b, h, I) from the item index w ----
  auto run_item = [&](const int w) {
    const FaItem it = fa_item(w, gp, G, Nb, nbg);
    const int bg = it.bg, hh = it.hh, I = it.I;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int h = g * G + hh;
    const int64_t row = (static_cast<int64_t>(b) * H + h) * Nb + I;

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int lane = tid & 63;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int q_local = wv * 32 + col;  // query inside the block
    const int64_t q_tok = static_cast<int64_t>(I) * BLK + q_local;

    // Q as the B operand of S^T = K Q^T: 8 consecutive channels per lane and chunk.
    bf16x8 qb[C::KC];
    {
      const int64_t q_ld = q_tok < L ? q_tok : L - 1;  // rows beyond a ragged end: loaded, never stored
      const uint16_t* qrow = q + ((static_cast<int64_t>(b) * H + h) * L + q_ld) * D + half * 8;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) qb[kc] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + kc * 16));
    }
    // Complete the Q loads now (an empty asm consuming the registers makes the
    // compiler wait here): inside the loop vmcnt also counts the K/V copies in
    // flight, so a compiler-placed wait for Q there would drain the prefetch.
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) asm volatile("" ::"v"(qb[kc]));

    // One pass over the item's key blocks, with the reference max of each row
    // fixed by its first sub-tile (fast = true) or the exact running max.
    // Returns false, having stored nothing, when the fast pass's denominators
    // left [0, 2^64].  (A runtime flag, not a template: one copy of the loop.)
    auto pass = [&](const bool fast) -> bool {
      if (fast && threadIdx.x == 0) s_redo = 0;
      floatx16 o[C::CT];
  #pragma unroll
      for (int ct = 0; ct < C::CT; ++ct)
  #pragma unroll
        for (int e = 0; e < 16; ++e) o[ct][e] = 0.0f;
      float m = -INFINITY;  // reference max (base-2 logits)
      float l = 0.0f;       // this lane half's share of the denominator (sum of the bf16 p)

      // The index list is read-only for the whole kernel: read it through the
      // constant address space so the uniform loads are scalar (s_load).
      const int nblk = (idx == nullptr) ? (causal ? I + 1 : Nb) : ((const_i32_ptr)(cnt))[row];
      const int n_sub = nblk * C::SUB;
      const_i32_ptr list = (idx == nullptr) ? nullptr : ((const_i32_ptr)(idx)) + row * Nb;
      const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k) + static_cast<int64_t>(bg) * L * C::ROWB;
      const uint8_t* vbase = reinterpret_cast<const uint8_t*>(v) + static_cast<int64_t>(bg) * L * C::ROWB;

      // Per-lane pieces of the copy addresses: lane -> (row inside the instruction's rows, chunk slot).
      const int cp_row = lane / C::RC;
      const int cp_slot = lane % C::RC;

      auto block_of = [&](int s) { return (list == nullptr) ? s / C::SUB : list[s / C::SUB]; };
      // Global byte offset (inside a sub-tile) of the 16 bytes this lane copies in
      // each of its copy instructions; the same for K and V.
      int goff[C::IPW];
      int grow[C::IPW];
  #pragma unroll
      for (int i = 0; i < C::IPW; ++i) {
        const int inst = wv * C::IPW + i;
        const int r = inst * C::ROWS_PER_INST + cp_row;
        const int chunk = cp_slot ^ (swz(r) & (C::RC - 1));
        goff[i] = r * C::ROWB + chunk * 16;
        grow[i] = r;
      }
      // Copy sub-tile t of K or V (block J) into an LDS buffer: IPW instructions per wave.
      auto copy_tile = [&](const uint8_t* base, int t, int J, uint8_t* buf) {
        const int key0 = J * BLK + (t % C::SUB) * C::KT;  // < L < 2^31
        const uint8_t* gtile = base + static_cast<int64_t>(key0) * C::ROWB;
        const uint32_t l0 = lds_addr(buf) + wv * C::IPW * 1024;
        if (key0 + C::KT <= L) {
          static_for<C::IPW>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            copy16_to_lds<i * 1024>(gtile, goff[i], l0);
          });
        } else {  // tail sub-tile of a ragged sequence: rows past the end repeat row L-1
          // (the lane offsets are unsigned, so they stay >= 0: rebase on row L-1
          // when the whole sub-tile lies past the end)
          const int last = L - 1 - key0;
          if (last >= 0) {
            static_for<C::IPW>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              const int over = grow[i] - last;
              copy16_to_lds<i * 1024>(gtile, over > 0 ? goff[i] - over * C::ROWB : goff[i], l0);
            });
          } else {
            const uint8_t* gend = base + static_cast<int64_t>(L - 1) * C::ROWB;
            static_for<C::IPW>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              copy16_to_lds<i * 1024>(gend, goff[i] - grow[i] * C::ROWB, l0);
            });
          }
        }
      };

      // LDS read offsets that do not depend on the sub-tile.
      int koff[C::KC];  // S^T A operand: key row 32t + col (t added later), chunk 2kc + half
      {
        const int sw = swz(col) & (C::RC - 1);
  #pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) koff[kc] = col * C::ROWB + (((2 * kc + half) ^ sw) * 16);
      }
      // V^T A operand via transposed reads: key row kb0 + s/4 with kb0 = 32t + 16u + 4 half (+8),
      // channel 32 ct + 16 g16 + 4 (s % 4) (+ lane's element).
      const int s16 = lane & 15;
      const int g16 = (lane >> 4) & 1;
      int voff[2][C::CT];
  #pragma unroll
      for (int e8 = 0; e8 < 2; ++e8) {
        const int r = 4 * half + 8 * e8 + (s16 >> 2);  // row bits below 16 (t, u add multiples of 16)
        const int sw = swz(r) & (C::RC - 1);
  #pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
          const int chunk = 4 * ct + 2 * g16 + ((s16 & 3) >> 1);
          voff[e8][ct] = r * C::ROWB + ((chunk ^ sw) * 16) + (s16 & 1) * 8;
        }
      }

      // S^T = K Q^T for the 64 keys of a K buffer.
      auto qk = [&](const uint8_t* kbuf, floatx16 (&st)[2]) {
  #pragma unroll
        for (int t = 0; t < 2; ++t) {
  #pragma unroll
          for (int e = 0; e < 16; ++e) st[t][e] = 0.0f;
  #pragma unroll
          for (int kc = 0; kc < C::KC; ++kc) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(kbuf + koff[kc] + 32 * t * C::ROWB);
            st[t] = mfma32x32x16(as_bf16x8(a), qb[kc], st[t]);
          }
        }
      };

      // The block whose keys need a mask, and the last visible key inside it.
      const int mask_blk = causal ? I : ((L % BLK != 0) ? Nb - 1 : -1);
      const int mask_lim = causal ? q_local : L - 1 - (Nb - 1) * BLK;

      // Pipeline over sub-tiles t = 0 .. n_sub-1 (block J(t) = block_of(t)).  K runs
      // one sub-tile ahead of V: iteration s computes S(s+1) = K(s+1) Q^T with the
      // MFMA unit while the VALU turns S(s) into probabilities, then O += V(s) P(s).
      // Copies issued in iteration s: V(s+1) and K(s+2), into the buffers that held
      // V(s-1) and K(s), both consumed before the previous closing barrier.
      // Scores of the current and the next sub-tile, swapped between the two
      // unrolled steps of the loop (no register copies).
      floatx16 st_a[2], st_b[2];
      int J_cur = 0, J_n1 = 0;
      if (n_sub > 0) {
        J_cur = block_of(0);
        copy_tile(kbase, 0, J_cur, kb0);
        copy_tile(vbase, 0, J_cur, vb0);
        if (n_sub > 1) {
          J_n1 = block_of(1);
          copy_tile(kbase, 1, J_n1, kb1);
          wait_vmcnt<2 * C::IPW>();
        } else {
          wait_vmcnt<C::IPW>();
        }
        lds_barrier();  // K(0) landed for every wave
        qk(kb0, st_a);
        lds_reads_done_barrier();  // every wave has read K(0) before step 0 refills kb0 with K(2)
      }

      auto step = [&](int s, const uint8_t* kcur, const uint8_t* vcur, uint8_t* knext, uint8_t* vnext,
                      floatx16 (&st_cur)[2], floatx16 (&st_next)[2]) {
        // kcur = K(s+1), vcur = V(s); V(s+1) -> vnext, K(s+2) -> knext.
        int J_n2 = J_n1;
        if (s + 2 < n_sub) {
          J_n2 = block_of(s + 2);
          copy_tile(vbase, s + 1, J_n1, vnext);
          copy_tile(kbase, s + 2, J_n2, knext);
          wait_vmcnt<2 * C::IPW>();
        } else if (s + 1 < n_sub) {
          copy_tile(vbase, s + 1, J_n1, vnext);
          wait_vmcnt<C::IPW>();
        } else {
          wait_vmcnt<0>();
        }
        lds_barrier();  // V(s) and K(s+1) landed for every wave

        // Mask of S(s) in the one block that needs it (rare; own branch): the
        // diagonal block when causal, else the last block of a ragged sequence.
        if (J_cur == mask_blk) {
          const int key_base = (s % C::SUB) * C::KT;
  #pragma unroll
          for (int t = 0; t < 2; ++t)
  #pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key_local = key_base + 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
              if (key_local > mask_lim) st_cur[t][e] = -INFINITY;
            }
        }

        // ---- S(s+1) on the MFMA unit, softmax of S(s) on the VALU ----
        // Row max of S(s) first (it gates every exponential): on every sub-tile
        // in the exact pass, on the first one only in the fast pass.
        bool raise = false;
        float m_new = m;
        if (!fast || s == 0) {
          float mx = -INFINITY;
  #pragma unroll
          for (int t = 0; t < 2; ++t)
  #pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st_cur[t][e]);
          mx = max_halves(mx) * c;
          raise = mx > m;  // m = -inf on the first sub-tile
          m_new = raise ? mx : m;
        }
        // 16 chunks, each one MFMA of S(s+1) = K(s+1) Q^T (MFMA i: key tile i / KC,
        // k-chunk i % KC), one probability pair of S(s), and the LDS read of the
        // K fragment four MFMAs ahead, left for the compiler to interleave (a
        // scheduling barrier after every chunk measured 0.6 % slower).  (For the
        // last sub-tile the product re-reads a stale K buffer; its result is unused.)
  #pragma unroll
        for (int t = 0; t < 2; ++t)
  #pragma unroll
          for (int e = 0; e < 16; ++e) st_next[t][e] = 0.0f;
        constexpr int NM = 2 * C::KC;  // MFMAs of one 64-key S^T tile
        constexpr int AHEAD = 4;
        u32x4 kf[NM];
        auto kfrag = [&](int i) {
          return *reinterpret_cast<const u32x4*>(kcur + koff[i % C::KC] + 32 * (i / C::KC) * C::ROWB);
        };
  #pragma unroll
        for (int i = 0; i < AHEAD; ++i) kf[i] = kfrag(i);
        // Higher issue priority for the interleaved MFMA / softmax stream than for
        // the other wave's P V burst on this SIMD (measured: 2 % faster sparse).
        __builtin_amdgcn_s_setprio(2);
        u32x4 pb[2][2];
        float lsum = 0.0f;
        constexpr int NCHUNK = NM > 16 ? NM : 16;  // 16 probability pairs per sub-tile
  #pragma unroll
        for (int i = 0; i < NCHUNK; ++i) {
          if (i + AHEAD < NM) kf[i + AHEAD] = kfrag(i + AHEAD);
          if (i < NM) st_next[i / C::KC] = mfma32x32x16(as_bf16x8(kf[i]), qb[i % C::KC], st_next[i / C::KC]);
          if (i < 16) {
            const int t = i >> 3, u = (i >> 2) & 1, e = i & 3;
            const float p0 = fast_exp2(fmaf(st_cur[t][8 * u + 2 * e], c, -m_new));
            const float p1 = fast_exp2(fmaf(st_cur[t][8 * u + 2 * e + 1], c, -m_new));
            pb[t][u][e] = pack_bf16x2(p0, p1);
            lsum = add_bf16x2(pb[t][u][e], lsum);  // the same rounded p as V^T P^T
          }
        }
        __builtin_amdgcn_s_setprio(0);
        // Keep the probabilities in this block (ahead of the rescale branch).
  #pragma unroll
        for (int t = 0; t < 2; ++t)
  #pragma unroll
          for (int u = 0; u < 2; ++u) asm volatile("" ::"v"(pb[t][u]));
        asm volatile("" ::"v"(lsum));

        if (!fast && __any(raise)) {
          const float alpha = fast_exp2(m - m_new);
          l *= alpha;
  #pragma unroll
          for (int ct = 0; ct < C::CT; ++ct)
  #pragma unroll
            for (int e = 0; e < 16; ++e) o[ct][e] *= alpha;
        }
        m = m_new;
        l += lsum;

        // ---- O^T += V^T P^T: 16 MFMAs, V^T fragments read AV MFMAs ahead ----
        constexpr int NP = 4 * C::CT;  // (t, u, ct) triples
        constexpr int AV = 3;
        u32x4 vf[NP];
        auto vfrag = [&](int j) {
          const int t = j / (2 * C::CT), u = (j / C::CT) & 1, ct = j % C::CT;
          const int rowoff = (32 * t + 16 * u) * C::ROWB;
          const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vcur + rowoff + voff[0][ct]));
          const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vcur + rowoff + voff[1][ct]));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
          return a;
        };
  #pragma unroll
        for (int j = 0; j < AV; ++j) vf[j] = vfrag(j);
  #pragma unroll
        for (int j = 0; j < NP; ++j) {
          if (j + AV < NP) vf[j + AV] = vfrag(j + AV);
          const int t = j / (2 * C::CT), u = (j / C::CT) & 1, ct = j % C::CT;
          o[ct] = mfma32x32x16(as_bf16x8(vf[j]), as_bf16x8(pb[t][u]), o[ct]);
          __builtin_amdgcn_sched_barrier(0);
        }
        lds_reads_done_barrier();  // every wave is done with K(s+1)'s and V(s)'s buffers
        J_cur = J_n1;
        J_n1 = J_n2;
      };
      for (int s = 0; s < n_sub; s += 2) {
        step(s, kb1, vb0, kb0, vb1, st_a, st_b);
        if (s + 1 < n_sub) step(s + 1, kb0, vb1, kb1, vb0, st_b, st_a);
      }

      // ---- normalise and store: lane holds 4 consecutive channels per group ----
      l = sum_halves(l);
      if (fast) {  // every wave learns whether any row of the item left the range
        if (__any(!(l <= 0x1p64f)) && lane == 0) s_redo = 1;
        __syncthreads();
        const int redo = s_redo;
        __syncthreads();
        if (redo) return false;
      }
      const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
      uint16_t* orow = out + ((static_cast<int64_t>(b) * H + h) * L + q_tok) * D;
      if (q_tok >= L) return true;  // past a ragged end
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
      return true;
    };  // pass
    bool fast = true;
    while (!pass(fast)) fast = false;  // at most twice: the exact pass always stores
  };  // run_item

  // ---- items: blockIdx.x alone, or popped from the XCD queues ----
  const int n_items = nbg * G * Nb;
  const int x0 = blockIdx.x % kSchedQueues;
  int tries = 0;  // queues thread 0 has found empty, in the order x0, x0 + 1, ...
  auto pop = [&]() -> int {
    if (threadIdx.x == 0) {
      int it = -1;
      while (tries < kSchedQueues) {
        const int x = (x0 + tries) % kSchedQueues;
        const int n_x = (n_items - x + kSchedQueues - 1) / kSchedQueues;  // items w = 8k + x < n_items
        const uint32_t kq = atomicAdd(&sched[kSchedStride * x], 1u);
        if (kq < static_cast<uint32_t>(n_x)) {
          it = kSchedQueues * static_cast<int>(kq) + x;
          break;
        }
        ++tries;
      }
      s_item = it;
    }
    __syncthreads();
    const int it = s_item;
    __syncthreads();  // every thread has read s_item before thread 0 rewrites it
    return it;
  };
  int item = (sched == nullptr) ? static_cast<int>(blockIdx.x) : pop();
  while (item >= 0) {
    run_item(item);
    item = (sched == nullptr) ? -1 : pop();
  }
}

// Clears the schedule counters (a kernel, not a memset, so the launch can be
// captured in a graph).
__global__ void sched_clear_kernel(uint32_t* __restrict__ sched) {
  for (int i = threadIdx.x; i < kSchedQueues * kSchedStride; i += blockDim.x) sched[i] = 0u;
}

static int phase_groups(const Shape& s, int64_t budget) {
  return fa_phase_groups(s.Bz * s.Hkv, s.Nb, int64_t(2) * s.L * s.d * 2, budget);
}

// Workgroups of flash_attn_kernel<D, BLK> resident at once on the current
// device (occupancy x CUs), 0 if unknown; cached per device and kernel.
template <int D, int BLK>
static int resident_workgroups() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, flash_attn_kernel<D, BLK>, FaCfg<D, BLK>::NT, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  n = per_cu * cus;
  n -= n % kSchedQueues;  // whole rounds over the XCDs
  if (n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int BLK>
static int launch_fa(const Shape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                     const int32_t* cnt, uint16_t* out, uint32_t* sched, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(s.Bz) * s.H * s.Nb;
  int64_t grid = items;
  if (sched != nullptr) {
    const int resident = resident_workgroups<D, BLK>();
    if (resident > 0 && items > resident) {
      hipLaunchKernelGGL(sched_clear_kernel, dim3(1), dim3(256), 0, st, sched);
      const int err = static_cast<int>(hipGetLastError());
      if (err != 0) return err;
      grid = resident;
    } else {
      sched = nullptr;  // every item has a workgroup of its own anyway
    }
  }
  hipLaunchKernelGGL((flash_attn_kernel<D, BLK>), dim3(static_cast<unsigned>(grid)), dim3(FaCfg<D, BLK>::NT), 0,
                     st, q, k, v, idx, cnt, out, s.H, s.Hkv, s.G, s.L, s.Nb, s.scale * kLog2e,
                     phase_groups(s, idx != nullptr ? kSparsePhaseBytes : kDensePhaseBytes), s.causal ? 1 : 0,
                     s.Bz * s.Hkv, sched);
  return static_cast<int>(hipGetLastError());
}

int launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                      const int32_t* cnt, uint16_t* out, uint32_t* sched, void* stream) {
  if (static_cast<int64_t>(s.Bz) * s.Nb == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.d == 128 && s.Bk == 128) return launch_fa<128, 128>(s, q, k, v, idx, cnt, out, sched, st);
  if (s.d == 128 && s.Bk == 64) return launch_fa<128, 64>(s, q, k, v, idx, cnt, out, sched, st);
  if (s.d == 64 && s.Bk == 128) return launch_fa<64, 128>(s, q, k, v, idx, cnt, out, sched, st);
  return launch_fa<64, 64>(s, q, k, v, idx, cnt, out, sched, st);
}

}  // namespace rra
