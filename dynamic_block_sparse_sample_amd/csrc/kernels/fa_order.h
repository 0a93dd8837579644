// Work order of the attention kernel: which (KV row, head, query block) item w
// is, and how many KV groups share a phase.  Plain constexpr C++ (callable from
// the kernel and from host code), so the mapping can be checked on the CPU.
#ifndef RRA_FA_ORDER_H_
#define RRA_FA_ORDER_H_

#include <cstdint>

namespace rra {

// Phase budgets (bytes of K and V of the groups in one phase), measured on the
// 32K / 64K / 128K workloads: dense launches read each group's K and V in step
// across its rows and do best with phases of up to half the 256 MB
// memory-side cache; sparse launches re-read K/V blocks scattered by their
// lists and do best with a quarter (at 128K one group per phase: sparse 1.2 %
// faster, dense 0.8 % slower than with two).
constexpr int64_t kDensePhaseBytes = int64_t(128) << 20;
constexpr int64_t kSparsePhaseBytes = int64_t(64) << 20;

// Groups per phase: the largest gp in {8, 4, 2, 1} that divides the group
// count nbg, splits the Nb query blocks evenly over 8/gp XCDs and keeps gp
// groups' K and V (kv_bytes each) within the budget; one group per phase above
// the budget when Nb is a multiple of 8, else 0 (plain order).
constexpr int fa_phase_groups(int nbg, int Nb, int64_t kv_bytes, int64_t budget) {
  for (int gp = 8; gp >= 1; gp >>= 1) {
    if (nbg % gp == 0 && Nb % (8 / gp) == 0 && gp * kv_bytes <= budget) return gp;
  }
  return Nb % 8 == 0 ? 1 : 0;
}

struct FaItem {
  int bg;  // b * Hkv + g
  int hh;  // head inside the group (h = g * G + hh)
  int I;   // query block
};

// Item w (run on XCD w mod 8).  With gp > 0 the KV groups are processed in
// phases of gp groups (their K and V fit the memory-side cache together);
// inside a phase XCD x takes every (8/gp)-th query block, longest rows first,
// the G heads of a group in consecutive slots (they stream the same K/V
// through the XCD's L2).  The group an XCD serves rotates every 16 slots
// (about the workgroups an XCD holds at once, so neighbouring query blocks of
// a group, whose lists overlap, still share the L2): groups differ in density,
// and a fixed assignment would leave the XCDs of the sparser groups idle at the
// end.  gp = 0: heads, then groups, then query blocks from the last.
constexpr FaItem fa_item(int w, int gp, int G, int Nb, int nbg) {
  FaItem it{0, 0, 0};
  if (gp > 0) {
    const int phase_items = gp * G * Nb;
    const int ph = w / phase_items;
    const int r = w % phase_items;
    const int xcd = r & 7;
    int slot = r >> 3;
    const int split = 8 / gp;
    it.hh = slot % G;
    slot /= G;
    it.I = Nb - 1 - (slot * split + xcd / gp);
    it.bg = ph * gp + (xcd + (slot >> 4)) % gp;
  } else {
    int t = w;
    it.hh = t % G;
    t /= G;
    it.bg = t % nbg;
    it.I = Nb - 1 - t / nbg;
  }
  return it;
}

}  // namespace rra

#endif  // RRA_FA_ORDER_H_
