// Host build of the schedule functions the main kernel evaluates per tile
// (csrc/tile_sched.h), compiled with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py. For every schedule,
// mask, tile ratio, KV-tile count and ring size it walks every item the way
// the kernel does (SegWalk) and checks, with no undefined behaviour on the way:
//  * each step equals the closed forms Sched::tile and Sched::rank;
//  * the items cover every visible (Q tile, KV tile) pair exactly once;
//  * each dQ tile's ranks are 0, 1, ..., count-1 (a fixed total order).
// Prints "ok <cases>" or the first mismatch, and exits non-zero on a failure.
#define __host__
#define __device__
#define __forceinline__ inline
#include "tile_sched.h"

#include <cstdio>
#include <vector>

using namespace detattn;

static int check(int sch, int causal, int n_kv, int r, int G) {
  const int n_q = n_kv * r;
  Sched sc{sch, causal, n_q, n_kv, r, G};
  const int ip = sc.items_per_head();
  std::vector<int> seen((size_t)n_q * n_kv, 0);
  std::vector<std::vector<int>> ranks(n_q);
  for (int it = 0; it < ip; ++it) {
    for (int seg = 0; seg < sc.segments(); ++seg) {
      int j = -1;
      SegWalk w = sc.walk(it, seg, j);
      for (int t = sc.seg_begin(it, seg); t < sc.seg_end(it, seg); ++t) {
        if (t > sc.seg_begin(it, seg)) w.advance(t);
        int ci, cj;
        sc.tile(it, t, ci, cj);
        if (ci != w.i || cj != j || ci < 0 || ci >= n_q || cj < 0 || cj >= n_kv) {
          std::printf("walk mismatch sch %d causal %d n_kv %d r %d G %d item %d step %d: (%d,%d) vs (%d,%d)\n", sch,
                      causal, n_kv, r, G, it, t, w.i, j, ci, cj);
          return 1;
        }
        if (sch != kAtomicNondet) {
          const int rk = w.rank_now();
          if (rk != sc.rank(ci, cj)) {
            std::printf("rank mismatch sch %d n_kv %d r %d G %d item %d step %d: %d vs %d\n", sch, n_kv, r, G, it, t,
                        rk, sc.rank(ci, cj));
            return 1;
          }
          ranks[ci].push_back(rk);
        }
        ++seen[(size_t)ci * n_kv + cj];
      }
    }
  }
  for (int i = 0; i < n_q; ++i)
    for (int j = 0; j < n_kv; ++j) {
      const int want = (!causal || i >= j * r) ? 1 : 0;  // Q tile i sees KV tile j unless it lies wholly above
      if (seen[(size_t)i * n_kv + j] != want) {
        std::printf("coverage sch %d causal %d n_kv %d r %d G %d: tile (%d,%d) visited %d times\n", sch, causal, n_kv,
                    r, G, i, j, seen[(size_t)i * n_kv + j]);
        return 1;
      }
    }
  for (int i = 0; i < n_q && sch != kAtomicNondet; ++i) {
    std::vector<int> hit(ranks[i].size(), 0);
    for (int rk : ranks[i]) {
      if (rk < 0 || rk >= (int)hit.size() || hit[rk]++) {
        std::printf("ranks of dQ tile %d not a permutation (sch %d n_kv %d r %d G %d)\n", i, sch, n_kv, r, G);
        return 1;
      }
    }
  }
  return 0;
}

int main() {
  int cases = 0;
  const int kvs[] = {1, 2, 3, 4, 6, 8, 10, 16, 37, 40, 64};
  for (int sch = 0; sch <= 4; ++sch)
    for (int causal = 0; causal <= 1; ++causal)
      for (int n_kv : kvs)
        for (int r : {1, 2, 4}) {
          if (sch == kShift && causal) continue;
          if (sch == kSymmetricShift && (!causal || n_kv % 2)) continue;
          Sched probe{sch, causal, n_kv * r, n_kv, r, 0};
          const int ip = probe.items_per_head();
          const bool rings = sch == kShift || sch == kSymmetricShift;
          for (int G = rings ? 1 : 0; G <= (rings ? ip : 0); ++G) {
            if (G > 0 && ip % G) continue;
            if (check(sch, causal, n_kv, r, G)) return 1;
            ++cases;
          }
        }
  std::printf("ok %d\n", cases);
  return 0;
}
