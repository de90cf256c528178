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
        const int i = cnt[x].fetch_add(chunk, std::memory_order_relaxed);
        if (i >= n) break;
        for (int v = begin + i; v < begin + (i + chunk < n ? i + chunk : n); ++v) {
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

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string mode = argv[1];
  if (mode == "static" && argc == 7)
    return static_walk(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                       std::atoi(argv[6]));
  if (mode == "ws" && argc == 8)
    return ws_threads(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                      std::atoi(argv[6]), std::atoi(argv[7]));
  return 2;
}
