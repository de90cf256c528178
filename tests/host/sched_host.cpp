// Host build of the library's scheduler header (csrc/sched.hpp): prints the
// schedule every program walks, and runs the work-stealing claim loop with
// std::atomic counters on real threads.  Output is compared by
// tests/test_sched_host.py against the oracle's schedule model.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <thread>
#include <vector>

#include "../../tile_scheduling_persistent_amd/csrc/sched.hpp"

static int static_walk(int kind, int pm, int pn, int G, int gs) {
  const int T = pm * pn;
  for (int p = 0; p < G; ++p) {
    int v, end;
    pgs::static_first(kind, p, T, G, v, end);
    std::printf("%d:", p);
    while (v < end) {
      int m, n;
      pgs::decode(kind, v, pm, pn, gs, m, n);
      std::printf(" %d,%d,%d", v, m, n);
      v = pgs::static_next(kind, v, G, end);
    }
    std::printf("\n");
  }
  return 0;
}

// One claim on `c` for a range of n tiles: [first, end) relative to the
// range's start, or false when the range is exhausted.  chunk < 0: paired
// claims (the counter counts claims, pgs::pair_claim maps them to tiles).
static bool take(std::atomic<int>& c, int n, int chunk, int G, int X, int& first, int& end) {
  if (chunk < 0) {
    const int k = c.fetch_add(1, std::memory_order_relaxed);
    return pgs::pair_claim(k, n, G, X, first, end);
  }
  const int i = c.fetch_add(chunk, std::memory_order_relaxed);
  first = i;
  end = i + chunk < n ? i + chunk : n;
  return i < n;
}

// G threads claim from X atomic counters exactly as the kernels do.
static int ws_threads(int pm, int pn, int G, int X, int gs, int chunk) {
  const int T = pm * pn;
  std::vector<std::atomic<int>> cnt(X);
  for (auto& c : cnt) c.store(0);
  std::vector<std::atomic<int>> visits(T);
  for (auto& v : visits) v.store(0);
  std::vector<int> owner(T, -1), order(T, -1);
  std::vector<std::thread> th;
  for (int p = 0; p < G; ++p) {
    th.emplace_back([&, p] {
      const int x = p % X;
      const int begin = pgs::ws_range_begin(x, T, X);
      const int n = pgs::ws_range_begin(x + 1, T, X) - begin;
      int done = 0;
      for (;;) {
        int f, e;
        if (!take(cnt[x], n, chunk, G, X, f, e)) break;
        for (int v = begin + f; v < begin + e; ++v) {
          visits[v].fetch_add(1);
          owner[v] = p;
          order[v] = done++;
          std::this_thread::yield();
        }
      }
    });
  }
  for (auto& t : th) t.join();
  std::printf("counters:");
  for (int x = 0; x < X; ++x) std::printf(" %d", cnt[x].load());
  std::printf("\n");
  for (int v = 0; v < T; ++v) std::printf("%d %d %d %d\n", v, visits[v].load(), owner[v], order[v]);
  return 0;
}

// Work stealing across XCDs: G threads start on counter homes[p]; after a
// failing claim a thread reads the counters it has not passed (cyclic order),
// skips those past their range and moves to the first that is not, or stops;
// the end of a claim is cut at the end of the range that holds its first
// tile (pgs::ws_owner), as the kernels do.
static int wsx_threads(int pm, int pn, int G, int X, int chunk, int home_mode) {
  const int T = pm * pn;
  std::vector<int> homes(G);
  unsigned lcg = 12345u;
  for (int p = 0; p < G; ++p) {
    lcg = lcg * 1103515245u + 12345u;
    homes[p] = home_mode == 0 ? p % X : home_mode == 1 ? 0 : (int)((lcg >> 16) % (unsigned)X);
  }
  std::vector<std::atomic<int>> cnt(X);
  for (auto& c : cnt) c.store(0);
  std::vector<std::atomic<int>> visits(T);
  for (auto& v : visits) v.store(0);
  std::vector<int> owner(T, -1), order(T, -1);
  std::vector<std::thread> th;
  for (int p = 0; p < G; ++p) {
    th.emplace_back([&, p] {
      int x = homes[p], passed = 0, done = 0;
      auto range_n = [&](int c) { return pgs::ws_range_begin(c + 1, T, X) - pgs::ws_range_begin(c, T, X); };
      for (;;) {
        const int begin = pgs::ws_range_begin(x, T, X);
        const int n = range_n(x);
        int f, e;
        if (!take(cnt[x], n, chunk, G, X, f, e)) {
          if (++passed >= X) break;
          const int left = X - passed;
          std::vector<int> seen(left);
          for (int j = 0; j < left; ++j) seen[j] = cnt[(x + 1 + j) % X].load(std::memory_order_relaxed);
          auto claims_of = [&](int m) { return chunk < 0 ? pgs::pair_claims(m, G, X) : m; };
          int j = 0;
          while (j < left && seen[j] >= claims_of(range_n((x + 1 + j) % X))) ++j;
          if (j == left) break;
          passed += j;
          x = (x + 1 + j) % X;
          continue;
        }
        // the end is cut at the end of the range holding the first tile
        const int v0 = begin + f;
        const int range_end = pgs::ws_range_begin(pgs::ws_owner(v0, T, X) + 1, T, X);
        const int ve = begin + e < range_end ? begin + e : range_end;
        for (int v = v0; v < ve; ++v) {
          visits[v].fetch_add(1);
          owner[v] = p;
          order[v] = done++;
          std::this_thread::yield();
        }
      }
    });
  }
  for (auto& t : th) t.join();
  std::printf("homes:");
  for (int p = 0; p < G; ++p) std::printf(" %d", homes[p]);
  std::printf("\ncounters:");
  for (int x = 0; x < X; ++x) std::printf(" %d", cnt[x].load());
  std::printf("\n");
  for (int v = 0; v < T; ++v) std::printf("%d %d %d %d\n", v, visits[v].load(), owner[v], order[v]);
  return 0;
}

// Stream-K: every program's segments (tile, first slab, end slab, slot), then
// for every split tile its contributors with the slots they wrote.
static int sk_walk(int T, int nk, int G) {
  for (int p = 0; p < G; ++p) {
    pgs::SkWalker w;
    w.init(p, T, G, nk);
    std::printf("%d:", p);
    int v, kb, ke, slot;
    while (w.next(v, kb, ke, slot)) std::printf(" %d,%d,%d,%d", v, kb, ke, slot);
    std::printf("\n");
  }
  const int dp = pgs::sk_dp_tiles(T, G);
  const int64_t W = (int64_t)(T - dp) * nk;
  for (int v = dp; v < T; ++v) {
    const int64_t j0 = (int64_t)(v - dp) * nk;
    const int q0 = pgs::sk_owner(j0, W, G), q1 = pgs::sk_owner(j0 + nk - 1, W, G);
    if (q0 == q1) continue;
    std::printf("split %d:", v);
    for (int q = q0; q <= q1; ++q)
      if (pgs::sk_run_begin(q, W, G) < pgs::sk_run_begin(q + 1, W, G))  // empty runs add nothing
        std::printf(" %d,%d", q, pgs::sk_slot(q, v, dp, nk, W, G));
    std::printf("\n");
  }
  return 0;
}

// Paired-claim map for ranges of 0..139 tiles: n, L, claims, then each
// claim's first and end.
static int pairs_map(int G, int X) {
  for (int n = 0; n < 140; ++n) {
    const int claims = pgs::pair_claims(n, G, X);
    std::printf("%d %d %d", n, pgs::pair_span(n, G, X), claims);
    for (int k = 0; k < claims; ++k) {
      int f, e;
      if (!pgs::pair_claim(k, n, G, X, f, e)) return 1;
      std::printf(" %d %d", f, e);
    }
    std::printf("\n");
  }
  return 0;
}

// Default GEMM grid for T = 0..Tmax tiles: T and the balanced grid.
static int grid_map(int Tmax, int G, int X) {
  for (int T = 0; T <= Tmax; ++T) std::printf("%d %d\n", T, pgs::balanced_grid(T, G, X));
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string mode = argv[1];
  if (mode == "static" && argc == 7)
    return static_walk(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                       std::atoi(argv[6]));
  if (mode == "ws" && argc == 8)
    return ws_threads(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                      std::atoi(argv[6]), std::atoi(argv[7]));
  if (mode == "wsx" && argc == 8)
    return wsx_threads(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                       std::atoi(argv[6]), std::atoi(argv[7]));
  if (mode == "pairs" && argc == 4) return pairs_map(std::atoi(argv[2]), std::atoi(argv[3]));
  if (mode == "grid" && argc == 5) return grid_map(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]));
  if (mode == "sk" && argc == 5)
    return sk_walk(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]));
  return 2;
}
