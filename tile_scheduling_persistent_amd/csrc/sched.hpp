// Tile schedulers of the persistent kernels: integer functions shared by host
// and device code.  No memory access happens here; the work-stealing claim
// itself (one atomic on the XCD's counter) lives in the kernels.
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
//    XCD, chosen by program id modulo the XCD count.
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
};

PGS_FN int cdiv(int a, int b) { return (a + b - 1) / b; }

PGS_FN bool grouped_order(int kind) {
  return kind == kGrouped || kind == kWorkStealing || kind == kBlockedGrouped;
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

// Work stealing: XCD x owns tile ids [range_begin(x), range_begin(x + 1)).
PGS_FN int ws_range_begin(int x, int T, int X) {
  return (int)(((int64_t)x * (int64_t)T) / (int64_t)X);
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

}  // namespace pgs
