// CPU model of the main kernel's dispatch and ordered dQ hand-off (test
// infrastructure). Threads stand in for workgroups and std::atomic words for
// the per-dQ-tile flags in global memory. Every thread claims items as the
// kernel does (ticket counter in (head, item) order, or static rings whose
// slots take one item per round, odd rounds reversed in snake order), and for
// each tile waits until the dQ tile's flag equals the tile's rank, adds its
// partial (the first contributor stores), then publishes rank + 1. Waits are
// bounded; a timeout sets an error word that makes every later waiter give up,
// so the run always ends.
//
// stdin:  BH ipH n_q mode G rings snake threads seed drop_item timeout_ms
//         then, per item of a head: L, followed by L pairs (q_tile rank)
// stdout: "TIMEOUT", or "OK" and the accumulator bits of every (head, q_tile)
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

struct Tile {
  int i, rank;
};

// the partial of (head, item, step): a float with a full mantissa over eight
// binades, so that another summation order gives other bits
static float partial(int h, int item, int t) {
  uint32_t x = (uint32_t)h * 0x9E3779B1u ^ (uint32_t)(item + 1) * 0x85EBCA77u ^ (uint32_t)(t + 7) * 0xC2B2AE3Du;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  const float mant = 1.0f + (float)(x & 0x7FFFFF) / (float)(1 << 23);
  const int ex = (int)((x >> 23) % 8) - 4;
  const float v = std::ldexp(mant, ex);
  return (x >> 31) ? -v : v;
}

int main() {
  int BH, ipH, n_q, mode, G, rings, snake, threads, drop_item;
  unsigned seed;
  long timeout_ms;
  if (std::scanf("%d %d %d %d %d %d %d %d %u %d %ld", &BH, &ipH, &n_q, &mode, &G, &rings, &snake, &threads, &seed,
                 &drop_item, &timeout_ms) != 11)
    return 2;
  std::vector<std::vector<Tile>> items(ipH);
  for (int it = 0; it < ipH; ++it) {
    int L;
    if (std::scanf("%d", &L) != 1) return 2;
    items[it].resize(L);
    for (auto& tl : items[it])
      if (std::scanf("%d %d", &tl.i, &tl.rank) != 2) return 2;
  }
  std::vector<std::atomic<int>> flag(BH * n_q);
  std::vector<std::atomic<uint32_t>> acc(BH * n_q);
  for (auto& f : flag) f.store(0);
  for (auto& a : acc) a.store(0);
  std::atomic<long long> ticket{0};
  std::atomic<int> err{0};
  const long long total = (long long)BH * ipH;
  const auto deadline = std::chrono::milliseconds(timeout_ms);

  auto run = [&](int w) {
    std::mt19937 rng(seed * 7919u + (unsigned)w);
    std::uniform_int_distribution<int> coin(0, 7);
    auto jitter = [&]() {
      const int c = coin(rng);
      if (c == 0) std::this_thread::yield();
      else if (c == 1) std::this_thread::sleep_for(std::chrono::microseconds(coin(rng) * 20));
    };
    // ring state, as in the kernel
    const int ring_id = mode == 1 ? w / G : 0, slot = mode == 1 ? w % G : 0;
    if (mode == 1 && ring_id >= rings) return;
    int ring_bh = ring_id, ring_k0 = 0;
    bool ring_rev = false;
    for (;;) {
      long long g;
      if (mode == 0) {
        g = ticket.fetch_add(1);
        if (g >= total) return;
      } else {
        if (ring_bh >= BH) return;
        g = (long long)ring_bh * ipH + ring_k0 + (ring_rev ? G - 1 - slot : slot);
        ring_k0 += G;
        ring_rev = snake && !ring_rev;
        if (ring_k0 >= ipH) {
          ring_k0 = 0;
          ring_rev = false;
          ring_bh += rings;
        }
      }
      const int h = (int)(g / ipH), it = (int)(g % ipH);
      for (size_t t = 0; t < items[it].size(); ++t) {
        const Tile tl = items[it][t];
        const int f = h * n_q + tl.i;
        jitter();
        const auto t0 = std::chrono::steady_clock::now();
        while (flag[f].load(std::memory_order_acquire) != tl.rank) {
          if (err.load(std::memory_order_relaxed) || std::chrono::steady_clock::now() - t0 > deadline) {
            err.store(1);
            break;
          }
          std::this_thread::yield();
        }
        const float p = partial(h, it, (int)t);
        float sum = p;
        if (tl.rank > 0) {
          uint32_t bits = acc[f].load(std::memory_order_relaxed);
          float old;
          std::memcpy(&old, &bits, 4);
          sum = old + p;
        }
        uint32_t out;
        std::memcpy(&out, &sum, 4);
        acc[f].store(out, std::memory_order_relaxed);
        jitter();
        const bool withhold = (g == drop_item && t == 0);
        if (!withhold) flag[f].store(tl.rank + 1, std::memory_order_release);
      }
    }
  };
  std::vector<std::thread> pool;
  for (int w = 0; w < threads; ++w) pool.emplace_back(run, w);
  for (auto& th : pool) th.join();
  if (err.load()) {
    std::printf("TIMEOUT\n");
    return 0;
  }
  std::printf("OK\n");
  for (int f = 0; f < BH * n_q; ++f) std::printf("%08x\n", acc[f].load());
  return 0;
}
