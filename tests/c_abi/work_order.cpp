// CPU check of the attention kernel's work order (the header the kernel uses):
// for every shape below and both phase budgets, items 0 .. Bz*H*Nb-1 map onto
// every (KV row, head, query block) exactly once, inside its range; with
// phases, item w's query block sits on XCD w mod 8 in the phase's 8/gp-way
// split, the G heads of one (group, query block) take consecutive slots of one
// XCD, and each phase covers exactly its gp groups.  Prints "ok" and exits 0
// when every check holds.
#include <cstdio>
#include <vector>

#include "fa_order.h"

using rra::fa_item;
using rra::fa_phase_groups;

static int failures = 0;
#define EXPECT(cond, ...)                       \
  do {                                          \
    if (!(cond)) {                              \
      if (failures < 20) {                      \
        std::printf("FAIL %s: ", #cond);        \
        std::printf(__VA_ARGS__);               \
        std::printf("\n");                      \
      }                                         \
      ++failures;                               \
    }                                           \
  } while (0)

static void check(int Bz, int Hkv, int G, int L, int d, int Bk, long long budget, long long* n_checked) {
  const int Nb = (L + Bk - 1) / Bk;
  const int nbg = Bz * Hkv;
  const long long kv_bytes = 2LL * L * d * 2;
  const int gp = fa_phase_groups(nbg, Nb, kv_bytes, budget);
  EXPECT(gp == 0 || gp == 1 || gp == 2 || gp == 4 || gp == 8, "gp %d", gp);
  if (gp > 0) {
    EXPECT(nbg % gp == 0 && Nb % (8 / gp) == 0, "gp %d nbg %d Nb %d", gp, nbg, Nb);
    EXPECT(gp == 1 || gp * kv_bytes <= budget, "gp %d over budget", gp);
  }
  const long long n = static_cast<long long>(nbg) * G * Nb;
  std::vector<unsigned char> seen(static_cast<size_t>(n), 0);
  for (long long w = 0; w < n; ++w) {
    const rra::FaItem it = fa_item(static_cast<int>(w), gp, G, Nb, nbg);
    const bool in = it.bg >= 0 && it.bg < nbg && it.hh >= 0 && it.hh < G && it.I >= 0 && it.I < Nb;
    EXPECT(in, "shape %d/%d/%d/%d gp %d item %lld -> (%d, %d, %d)", Bz, Hkv, G, Nb, gp, w, it.bg, it.hh, it.I);
    if (!in) continue;
    const long long key = (static_cast<long long>(it.bg) * G + it.hh) * Nb + it.I;
    EXPECT(!seen[key], "shape %d/%d/%d/%d gp %d item %lld repeats (%d, %d, %d)", Bz, Hkv, G, Nb, gp, w, it.bg,
           it.hh, it.I);
    seen[key] = 1;
    if (gp > 0) {
      const int phase_items = gp * G * Nb;
      const int ph = static_cast<int>(w / phase_items);
      EXPECT(it.bg / gp == ph, "item %lld in phase %d serves group %d (gp %d)", w, ph, it.bg, gp);
      const int xcd = static_cast<int>(w % 8);
      EXPECT((Nb - 1 - it.I) % (8 / gp) == xcd / gp, "item %lld on XCD %d has block %d", w, xcd, it.I);
      // the G heads of one (group, block): slots G*k .. G*k+G-1 of this XCD
      const int slot = static_cast<int>((w % phase_items) >> 3);
      if (it.hh + 1 < G) {
        const rra::FaItem nx = fa_item(static_cast<int>(w + 8), gp, G, Nb, nbg);
        EXPECT(slot % G == it.hh && nx.bg == it.bg && nx.I == it.I && nx.hh == it.hh + 1,
               "item %lld: next head of (%d, %d) not in the next slot", w, it.bg, it.I);
      }
    }
  }
  for (long long key = 0; key < n; ++key) EXPECT(seen[key], "shape %d/%d/%d/%d gp %d misses %lld", Bz, Hkv, G, Nb, gp, key);
  *n_checked += n;
}

int main() {
  long long n_checked = 0;
  const long long budgets[] = {rra::kSparsePhaseBytes, rra::kDensePhaseBytes};
  for (long long budget : budgets) {
    // the workloads: tiny 1K, llama 8K / 32K / 128K, video 64K
    check(1, 4, 1, 1024, 64, 64, budget, &n_checked);
    check(1, 8, 4, 8192, 128, 128, budget, &n_checked);
    check(1, 8, 4, 32768, 128, 128, budget, &n_checked);
    check(1, 8, 4, 32768, 128, 64, budget, &n_checked);
    check(1, 8, 4, 131072, 128, 128, budget, &n_checked);
    check(1, 4, 7, 65536, 128, 128, budget, &n_checked);
    // a grid of batch, group counts, GQA ratios and lengths (ragged included)
    const int Bzs[] = {1, 2, 3};
    const int Hkvs[] = {1, 2, 3, 4, 8};
    const int Gs[] = {1, 2, 4, 7};
    const int Ls[] = {1, 64, 100, 640, 1000, 1024, 1025, 4096, 8192, 65536};
    const int ds[] = {64, 128};
    const int Bks[] = {64, 128};
    for (int Bz : Bzs)
      for (int Hkv : Hkvs)
        for (int G : Gs)
          for (int L : Ls)
            for (int d : ds)
              for (int Bk : Bks) check(Bz, Hkv, G, L, d, Bk, budget, &n_checked);
  }
  // The checker sees the mistake this order once had: 8 groups per phase
  // forced on 4 groups (video 64K) sends 7168 items past the last group.
  {
    int out = 0;
    for (int w = 0; w < 4 * 7 * 512; ++w) {
      const rra::FaItem it = fa_item(w, 8, 7, 512, 4);
      out += (it.bg >= 4) ? 1 : 0;
    }
    EXPECT(out == 7168, "forced gp = 8 on 4 groups: %d items out of range", out);
    EXPECT(fa_phase_groups(4, 512, 2LL * 65536 * 128 * 2, rra::kDensePhaseBytes) != 8, "gp 8 chosen for 4 groups");
  }
  std::printf("%lld items checked, %d failures\n", n_checked, failures);
  if (failures == 0) std::printf("ok\n");
  return failures == 0 ? 0 : 1;
}
