// Host build of the library's scheduler header (csrc/sched.hpp): prints the
// schedule every program walks, and runs the kernels' work-stealing claim
// loop (pgs::ws_claim) with std::atomic counters on real threads.  Output is compared by
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

// The counter operations the kernels perform with device atomics, on
// std::atomic counters: the claim loop itself is the library's
// (pgs::ws_claim), so these threads run the kernels' own claim and sweep code.
struct HostOps {
  std::atomic<int>* c;
  int* made;  // claims this thread made, per counter
  int fetch_add(int x, int v) {
    ++made[x];
    return c[x].fetch_add(v, std::memory_order_relaxed);
  }
  int load(int x) { return c[x].load(std::memory_order_relaxed); }
  void store(int x, int v) { c[x].store(v, std::memory_order_relaxed); }
};

// G threads walk the tiles as a kernel's programs do (Walker::first / next):
// a claim, the tiles of that claim in order, then the next claim, until a
// claim returns -1.  Thread p starts on counter homes[p]; `across` is work
// stealing across XCDs.  Prints the homes, the final counters, per tile its
// visits, owner and position in its owner's sequence, and last the claims
// each thread made on each counter (thread-major).
static int claim_threads(int pm, int pn, int G, int X, int chunk, bool across,
                         const std::vector<int>& homes, bool self_reset = false) {
  const int T = pm * pn;
  std::vector<std::atomic<int>> cnt(X);
  for (auto& c : cnt) c.store(0);
  std::vector<std::atomic<int>> visits(T);
  for (auto& v : visits) v.store(0);
  std::vector<int> owner(T, -1), order(T, -1);
  std::vector<int> made((size_t)G * X, 0);
  std::vector<std::thread> th;
  for (int p = 0; p < G; ++p) {
    th.emplace_back([&, p] {
      HostOps ops{cnt.data(), made.data() + (size_t)p * X};
      pgs::WsWalk w;
      pgs::ws_start(w, homes[p], T, X);
      const int reset_at = self_reset ? pgs::ws_last_claim_value(w.n, chunk, G, X, w.x) : -1;
      int done = 0;
      int v = pgs::ws_claim(w, across, T, G, X, chunk, ops, reset_at);
      while (v >= 0) {
        if (v >= T) std::abort();  // a claim past the tiles
        visits[v].fetch_add(1);
        owner[v] = p;
        order[v] = done++;
        std::this_thread::yield();
        v = v + 1 < w.cend ? v + 1 : pgs::ws_claim(w, across, T, G, X, chunk, ops, reset_at);
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
  std::printf("claims:");
  for (int m : made) std::printf(" %d", m);
  std::printf("\n");
  return 0;
}

// Per-XCD work stealing: program p claims from counter p mod X.
static int ws_threads(int pm, int pn, int G, int X, int chunk) {
  std::vector<int> homes(G);
  for (int p = 0; p < G; ++p) homes[p] = p % X;
  return claim_threads(pm, pn, G, X, chunk, false, homes);
}

// Per-XCD work stealing whose last failing claim on each counter zeroes it:
// prints each counter's reset value, then as ws_threads (the final counters
// should all be zero).
static int wsr_threads(int pm, int pn, int G, int X, int chunk) {
  const int T = pm * pn;
  std::printf("reset_at:");
  for (int x = 0; x < X; ++x) {
    const int n = pgs::ws_range_begin(x + 1, T, X) - pgs::ws_range_begin(x, T, X);
    std::printf(" %d", pgs::ws_last_claim_value(n, chunk, G, X, x));
  }
  std::printf("\n");
  std::vector<int> homes(G);
  for (int p = 0; p < G; ++p) homes[p] = p % X;
  return claim_threads(pm, pn, G, X, chunk, false, homes, true);
}

// Work stealing across XCDs from home counters p mod X (0), all 0 (1), or
// pseudo-random (2).
static int wsx_threads(int pm, int pn, int G, int X, int chunk, int home_mode) {
  std::vector<int> homes(G);
  unsigned lcg = 12345u;
  for (int p = 0; p < G; ++p) {
    lcg = lcg * 1103515245u + 12345u;
    homes[p] = home_mode == 0 ? p % X : home_mode == 1 ? 0 : (int)((lcg >> 16) % (unsigned)X);
  }
  return claim_threads(pm, pn, G, X, chunk, true, homes);
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

// Program numbering of the static walks: each workgroup id and the program
// it plays.
static int order_map(int G, int X, int xcd_major) {
  for (int hw = 0; hw < G; ++hw) std::printf("%d %d\n", hw, pgs::program_of(hw, G, X, xcd_major));
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string mode = argv[1];
  if (mode == "static" && argc == 7)
    return static_walk(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                       std::atoi(argv[6]));
  if (mode == "ws" && argc == 8)  // argv[6], the group size, does not enter the claims
    return ws_threads(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                      std::atoi(argv[7]));
  if (mode == "wsr" && argc == 7)
    return wsr_threads(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                       std::atoi(argv[6]));
  if (mode == "wsx" && argc == 8)
    return wsx_threads(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]),
                       std::atoi(argv[6]), std::atoi(argv[7]));
  if (mode == "pairs" && argc == 4) return pairs_map(std::atoi(argv[2]), std::atoi(argv[3]));
  if (mode == "grid" && argc == 5) return grid_map(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]));
  if (mode == "order" && argc == 5) return order_map(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]));
  if (mode == "sk" && argc == 5)
    return sk_walk(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]));
  return 2;
}
