// Tile schedulers of the persistent kernels: integer functions shared by host
// and device code.  No memory access happens here: the work-stealing claim
// loop (ws_claim) takes its counter operations from the caller (device
// atomics in the kernels, std::atomic in the host harness).
//
// Sources (page title, section):
//  - "Implement persistent kernels" (Helion PR #238), example output: blocked
//    ranges of cdiv(T, G) tiles per program, the stride-by-grid loop, the
//    decode with dimension 0 fastest, and the L2-grouped decode whose last
//    group is shortened by a min().
//  - "[Feature] Introduce tile scheduler" (TileLang PR #2441): a persistent
//    scheduler object with init / valid / next and a swizzle (group) size;
//    its loop walks tile ids with a stride of the grid.
//  - "Work Stealing Scheduler Kernel" (tritonBLAS PR #65): one counter per
//    XCD, chosen by program id modulo the XCD count (work stealing across
//    XCDs extends it: the home counter is the XCD the program runs on, and a
//    program whose home range is exhausted claims from the other counters in
//    cyclic order); stream-K is the
//    comparator its benchmark names (taken here as the data-parallel +
//    stream-K hybrid of the published Stream-K method).
#pragma once

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define PGS_FN __host__ __device__ __forceinline__
#else
#define PGS_FN inline
#endif

#include <stdint.h>

namespace pgs {

enum Kind : int {
  kBlocked = 0,
  kInterleaved = 1,
  kGrouped = 2,
  kWorkStealing = 3,
  kBlockedGrouped = 4,
  kStreamK = 5,
  kWorkStealingXcc = 6,
};

PGS_FN bool work_stealing(int kind) { return kind == kWorkStealing || kind == kWorkStealingXcc; }

PGS_FN int cdiv(int a, int b) { return (a + b - 1) / b; }

PGS_FN bool grouped_order(int kind) {
  return kind == kGrouped || kind == kWorkStealing || kind == kBlockedGrouped || kind == kStreamK ||
         kind == kWorkStealingXcc;
}

// Tile id -> (pid_m, pid_n), dimension 0 (rows of tiles) fastest.
PGS_FN void decode_plain(int v, int num_pid_m, int& pid_m, int& pid_n) {
  pid_m = v % num_pid_m;
  pid_n = v / num_pid_m;
}

// Grouped order: `gs` rows of tiles form a group that is walked column by
// column; the last group may hold fewer rows.
PGS_FN void decode_grouped(int v, int num_pid_m, int num_pid_n, int gs, int& pid_m,
                           int& pid_n) {
  const int in_group = gs * num_pid_n;
  const int group = v / in_group;
  const int first_m = group * gs;
  const int rows = (num_pid_m - first_m) < gs ? (num_pid_m - first_m) : gs;
  const int r = v - group * in_group;
  pid_m = first_m + r % rows;
  pid_n = r / rows;
}

PGS_FN void decode(int kind, int v, int num_pid_m, int num_pid_n, int gs, int& pid_m,
                   int& pid_n) {
  if (grouped_order(kind))
    decode_grouped(v, num_pid_m, num_pid_n, gs, pid_m, pid_n);
  else
    decode_plain(v, num_pid_m, pid_m, pid_n);
}

// Program numbering of the static walks.  The hardware hands the workgroups
// of a launch to the XCDs round robin (workgroup i to XCD (i + o) mod X, the
// start o depending on earlier launches), so workgroups with consecutive ids
// run on different XCDs and share no L2, and one XCD's workgroups are one
// residue class of i mod X.  XCD-major numbering gives the
// programs of one XCD consecutive ids: workgroup i plays program
// (i mod X) * (G / X) + i / X, and the neighbouring tiles of a static walk's
// round (which share operand panels) meet in one L2, as a work-stealing range
// does.  A bijection of [0, G); the identity unless xcd_major is set and
// X > 1 divides G.
PGS_FN int program_of(int hw, int G, int X, int xcd_major) {
  if (!xcd_major || X < 2 || G % X != 0) return hw;
  return (hw % X) * (G / X) + hw / X;
}

// Work stealing: XCD x owns tile ids [range_begin(x), range_begin(x + 1)).
PGS_FN int ws_range_begin(int x, int T, int X) {
  return (int)(((int64_t)x * (int64_t)T) / (int64_t)X);
}

// Default grid of the data-parallel GEMM schedulers: the fewest programs, a
// multiple of X, that finish in as many rounds of tiles as G programs do.
// The largest work-stealing range holds nx = ceil(T / X) tiles and its G / X
// programs take r = ceil(nx / (G / X)) rounds; ceil(nx / r) programs per XCD
// take the same r rounds, and so do the static walks (ceil(T / grid) <= r).
// The programs left out would only have idled through the last round, and
// with fewer CUs busy the busy ones run faster (measured on wave-quantised
// shapes).  G itself when T < 1, G < X or G is not a multiple of X.
PGS_FN int balanced_grid(int T, int G, int X) {
  if (T < 1 || X < 1 || G < X || G % X != 0) return G;
  const int nx = cdiv(T, X);
  const int r = cdiv(nx, G / X);
  return X * cdiv(nx, r);
}

// Paired claims (work-stealing option): the counter counts claims, and claim
// k of a range of n tiles takes tiles 2k, 2k+1 while k < L/2, then the single
// tile L + (k - L/2), where P = ceil(G / X) programs share a counter and
// L = 2 * min(n / 2, P * (ceil(n / P) / 2)): pairs for as many whole rounds of
// two as the range holds, so with equal speeds no program gets more tiles
// than with single claims.
PGS_FN int pair_span(int n, int G, int X) {
  const int P = cdiv(G, X);
  const int a = n / 2, b = P * (cdiv(n, P) / 2);
  return 2 * (a < b ? a : b);
}

PGS_FN int pair_claims(int n, int G, int X) {
  const int L = pair_span(n, G, X);
  return L / 2 + (n - L);
}

// Tiles [first, end) of claim k, relative to the range's start; false past
// the end of the range.
PGS_FN bool pair_claim(int k, int n, int G, int X, int& first, int& end) {
  const int L = pair_span(n, G, X);
  if (k < L / 2) {
    first = 2 * k;
    end = first + 2;
    return true;
  }
  first = L + (k - L / 2);
  end = first + 1;
  return first < n;
}

// Counter (XCD range) holding tile id v: the largest x with
// ws_range_begin(x) <= v.
PGS_FN int ws_owner(int v, int T, int X) {
  return (int)((((int64_t)v + 1) * X + T - 1) / T) - 1;
}

// Counters work stealing across XCDs can look at in one pass (the XCDs of
// one MI355X).
constexpr int kMaxStealCounters = 8;

// Claims a range of m tiles hands out (chunk < 0: paired claims).
PGS_FN int ws_claims_of(int m, int chunk, int G, int X) {
  return chunk < 0 ? pair_claims(m, G, X) : m;
}

// End (exclusive) of the claim of `chunk` tiles that starts at tile v, cut at
// the end of the counter range that holds v.
PGS_FN int ws_claim_end(int v, int chunk, int T, int X) {
  const int e = v + chunk;
  const int range_end = ws_range_begin(ws_owner(v, T, X) + 1, T, X);
  return e < range_end ? e : range_end;
}

// Programs whose home counter is x under per-XCD work stealing (p mod X).
PGS_FN int ws_programs_on(int x, int G, int X) { return G / X + (x < G % X ? 1 : 0); }

// Per-XCD work stealing: the value the last claim on counter x of one launch
// reads.  The counter's n tiles are handed out by a fixed number of
// successful claims, and each of the counter's programs then makes exactly
// one failing claim, so the launch's final counter value is known in advance
// and the claim that reads that value minus one step is the last operation on
// the counter in the launch.
PGS_FN int ws_last_claim_value(int n, int chunk, int G, int X, int x) {
  const int step = chunk < 0 ? 1 : chunk;
  const int claims = chunk < 0 ? pair_claims(n, G, X) : cdiv(n, chunk);
  return step * (claims + ws_programs_on(x, G, X) - 1);
}

// One program's position in the work-stealing walk.
struct WsWalk {
  int x;        // counter it claims from
  int passed;   // counters passed so far, the home counter first (across XCDs)
  int begin, n; // counter x's range [begin, begin + n)
  int cend;     // end (exclusive) of the last claim
};

PGS_FN void ws_set_counter(WsWalk& w, int c, int T, int X) {
  w.x = c;
  w.begin = ws_range_begin(c, T, X);
  w.n = ws_range_begin(c + 1, T, X) - w.begin;
}

PGS_FN void ws_start(WsWalk& w, int home, int T, int X) {
  w.passed = 0;
  w.cend = 0;
  ws_set_counter(w, home, T, X);
}

// One claim from counter w.x: `chunk` consecutive tiles, or under paired
// claims (chunk < 0) claim k's pair or single tile (pair_claim).  Work
// stealing across XCDs (across = true) goes on after a failing claim: it
// reads every counter it has not passed yet (one round of loads, cyclic order
// from w.x), skips those whose range is exhausted and claims from the first
// that is not; it stops when none is left, so it makes at most one failing
// claim per counter.  Returns the first claimed tile id and sets w.cend, or
// -1 when the program is done.  `ops` performs the memory operations on
// counter c: fetch_add(c, v) returns the old value, load(c) reads it, store(c,
// v) writes it (the kernels: device atomics, by one thread or by one lane for
// a whole wave; the host harness: std::atomic).  Needs X <= kMaxStealCounters
// when across.  reset_at >= 0 (per-XCD work stealing only): the failing claim
// that reads reset_at (ws_last_claim_value) stores zero into the counter, so
// the counters leave the launch as they entered it and the next launch needs
// no reset of its own.
template <class Ops>
PGS_FN int ws_claim(WsWalk& w, bool across, int T, int G, int X, int chunk, Ops& ops, int reset_at = -1) {
  for (;;) {
    const int step = chunk < 0 ? 1 : chunk;
    const int i = ops.fetch_add(w.x, step);
    if (chunk < 0) {
      int f, e;
      if (i >= 0 && pair_claim(i, w.n, G, X, f, e)) {
        w.cend = w.begin + e;
        return w.begin + f;
      }
    } else if (i >= 0 && i < w.n) {
      w.cend = ws_claim_end(w.begin + i, chunk, T, X);
      return w.begin + i;
    }
    if (!across) {
      if (i == reset_at) ops.store(w.x, 0);
      return -1;
    }
    if (++w.passed >= X) return -1;
    const int left = X - w.passed;
    int seen[kMaxStealCounters];
#if defined(__HIPCC__)
#pragma unroll
#endif
    for (int j = 0; j < kMaxStealCounters; ++j) {
      int c = w.x + 1 + j;
      c = c >= X ? c - X : c;
      seen[j] = j < left ? ops.load(c) : 0;
    }
    int j = 0;
    for (; j < left; ++j) {
      int c = w.x + 1 + j;
      c = c >= X ? c - X : c;
      if (seen[j] < ws_claims_of(ws_range_begin(c + 1, T, X) - ws_range_begin(c, T, X), chunk, G, X)) break;
    }
    if (j == left) return -1;
    w.passed += j;
    const int c = w.x + 1 + j;
    ws_set_counter(w, c >= X ? c - X : c, T, X);
  }
}

// Static schedulers: first tile id of program p and the end of its walk.
// A program whose first id is >= end computes nothing.
PGS_FN void static_first(int kind, int p, int T, int G, int& v, int& end) {
  if (kind == kBlocked || kind == kBlockedGrouped) {
    const int bs = cdiv(T, G);
    const int64_t s = (int64_t)p * bs;
    v = s < T ? (int)s : T;
    end = (s + bs) < T ? (int)(s + bs) : T;
  } else {  // interleaved, grouped
    v = p < T ? p : T;
    end = T;
  }
}

PGS_FN int static_step(int kind, int G) {
  return (kind == kBlocked || kind == kBlockedGrouped) ? 1 : G;
}

// Next tile id for static schedulers; returns a value >= end when done.
PGS_FN int static_next(int kind, int v, int G, int end) {
  const int64_t n = (int64_t)v + static_step(kind, G);
  return n < end ? (int)n : end;
}

// Stream-K.  T tiles of nk K-slabs on G programs.  Every full wave is
// data-parallel: the first floor(T/G)*G tiles (all of them when G divides
// T, none when T < G) are taken whole, stride-by-grid, and the
// W = (T - dp)*nk slabs of the remaining T mod G tiles are cut into G
// contiguous runs: program p takes slab indices [floor(p*W/G),
// floor((p+1)*W/G)) counted from tile dp.  A run is never longer than one
// tile, so it touches at most two tiles.  A tile whose slabs fall into
// several runs is finished from the runs' partial sums.
PGS_FN int sk_dp_tiles(int T, int G) { return (T / G) * G; }

PGS_FN int64_t sk_run_begin(int p, int64_t W, int G) { return ((int64_t)p * W) / G; }

// Program whose run holds stream-K slab index j (0 <= j < W).
PGS_FN int sk_owner(int64_t j, int64_t W, int G) {
  return (int)(((j + 1) * (int64_t)G + W - 1) / W) - 1;
}

// Partial-sum slot of program q for tile v (v in the stream-K part, split):
// 0 for the first tile of q's run, 1 for the second (a run touches at most
// two tiles).
PGS_FN int sk_slot(int q, int v, int dp, int nk, int64_t W, int G) {
  return (dp + (int)(sk_run_begin(q, W, G) / nk)) == v ? 0 : 1;
}

// The segments (tile, first slab, end slab) of one program, in order: its
// data-parallel tiles, then the pieces of its slab run.  slot is the
// partial-sum slot of a segment that does not cover its whole tile, -1
// otherwise.
struct SkWalker {
  int G, dp, nk;
  int64_t W;
  int v_dp;          // next data-parallel tile
  int64_t j, j_end;  // stream-K run cursor and end
  bool first;        // the next stream-K segment is the run's first

  PGS_FN void init(int p, int T, int G_, int nk_) {
    G = G_;
    nk = nk_;
    dp = sk_dp_tiles(T, G);
    W = (int64_t)(T - dp) * nk;
    v_dp = p;
    j = sk_run_begin(p, W, G);
    j_end = sk_run_begin(p + 1, W, G);
    first = true;
  }

  PGS_FN bool next(int& v, int& kb, int& ke, int& slot) {
    if (v_dp < dp) {
      v = v_dp;
      v_dp += G;
      kb = 0;
      ke = nk;
      slot = -1;
      return true;
    }
    if (j < j_end) {
      v = dp + (int)(j / nk);
      kb = (int)(j % nk);
      const int64_t left = j_end - j;
      ke = (int64_t)(nk - kb) < left ? nk : kb + (int)left;
      slot = (kb != 0 || ke != nk) ? (first ? 0 : 1) : -1;
      first = false;
      j += ke - kb;
      return true;
    }
    v = -1;
    kb = ke = 0;
    slot = -1;
    return false;
  }
};

}  // namespace pgs
