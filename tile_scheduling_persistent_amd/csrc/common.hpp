// Shared definitions of the HIP library: kernel parameter blocks, launcher
// declarations and the device-side tile walker used by every persistent
// kernel (GEMM bf16, GEMM block-scaled fp8, 2-D add).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sched.hpp"

namespace pgk {

// Optional instrumentation buffers (all NULL unless the witness is on).
struct Witness {
  int* visits;        // [T] times tile v was computed
  int* owner;         // [T] program that computed tile v
  int* order;         // [T] position of tile v in its owner's sequence
  long long* t_start; // [G] wall clock at program start
  long long* t_end;   // [G] wall clock at program end
  long long* cycles;  // [G] shader clock cycles from program start to end
  int* hw_id;         // [G] hardware placement of the program
  int* n_tiles;       // [G] tiles the program computed
  int* claims;        // [G][kMaxStealCounters] claims the program made on each counter
};

// Work-stealing counter x lives at counters[x * kCounterStride]: one 256-byte
// block per counter, so claims on different counters never contend for one
// cache line at the point where device-scope atomics are performed.
constexpr int kCounterStride = 64;
using pgs::kMaxStealCounters;

struct SchedParams {
  int kind;           // pgs::Kind
  int T;              // tiles
  int G;              // programs (grid)
  int X;              // XCDs = counters in use (work stealing)
  int gs;             // group size of the grouped order
  int num_pid_m;      // tiles along dimension 0 (rows)
  int num_pid_n;      // tiles along dimension 1 (columns)
  int* counters;      // work-stealing counters (stride kCounterStride), zero at launch
  int self_reset;     // per-XCD work stealing: the last failing claim on a counter zeroes it
  int xcd_major;      // static walks: programs numbered XCD-major (pgs::program_of)
  int chunk;          // tiles per work-stealing claim
  int straggler_program;  // -1: off
  int straggler_ns;
  int straggler_xcc;      // straggler_program names a hardware XCC, not a program
  int wall_khz;       // wall-clock tick rate (straggler wait)
};

// Several GEMMs in one launch: problem g owns the virtual tile ids
// [tile0, tile0 + npm * npn) of the shared space the scheduler walks.
constexpr int kMaxGemmProblems = 8;
struct GemmProblem {
  const void* A;   // [M][K]
  const void* B;   // [K][N]
  void* C;         // [M][N]
  const uint8_t* sa;  // fp8: e8m0 [K/128][M]
  const uint8_t* sb;  // fp8: e8m0 [K/128][N]
  int M, N, K;
  int tile0;       // first virtual tile id
  int npm, npn;    // tiles along M / N
};

struct GemmParams {
  const void* A;      // [M][K]
  const void* B;      // [K][N]
  void* C;            // [M][N]
  const uint8_t* sa;  // fp8: [K/128][M]
  const uint8_t* sb;  // fp8: [K/128][N]
  float* ws;          // stream-K: partial-sum slots [G][2][BM*BN] (fp32, tile-row-major)
  int M, N, K;
  SchedParams s;
  Witness w;
  int ngemm;          // several GEMMs: entries of gp in use (0: one problem, A..K above)
  GemmProblem gp[kMaxGemmProblems];
};

// Stream-K fix-up: the tiles whose slabs several programs shared are summed
// from the programs' partial-sum slots in slab order and written to C.
struct SkFixParams {
  const float* ws;
  void* C;
  int M, N;
  int T, nk, G, dp;
  long long W;
  int num_pid_m, num_pid_n, gs;
};

// Several adds in one launch: problem g owns the virtual tile ids
// [tile0, tile0 + npm * npn) of the shared space the scheduler walks.
constexpr int kMaxAddProblems = 8;
struct AddProblem {
  const float* X;
  const float* Y;
  float* C;
  int rows, cols;
  int tile0;     // first virtual tile id (prefix sum of the earlier problems' tiles)
  int npm, npn;  // tiles along rows / columns
};

struct AddParams {
  const float* X;
  const float* Y;
  float* C;
  int rows, cols;
  SchedParams s;
  Witness w;
  int nprob;     // several problems: 1..kMaxAddProblems entries of prob (0: X, Y, C above)
  AddProblem prob[kMaxAddProblems];
};

// Launchers: return hipErrorInvalidValue when no kernel is built for the
// requested tile shape.
hipError_t launch_gemm_bf16(const GemmParams& p, int bm, int bn, int bk, bool out_bf16,
                            bool vec, bool witness, hipStream_t stream);
hipError_t launch_gemm_fp8(const GemmParams& p, int bm, int bn, int bk, bool vec,
                           bool witness, hipStream_t stream);
hipError_t launch_padd(const AddParams& p, int tr, int tc, bool vec, bool witness,
                       hipStream_t stream);
hipError_t launch_padd_multi(const AddParams& p, int tr, int tc, bool vec, bool witness,
                             hipStream_t stream);
hipError_t launch_zero_i32(int* ptr, int n, hipStream_t stream);
hipError_t launch_fill_i32(int* ptr, int n, int value, hipStream_t stream);
bool gemm_bf16_tile_supported(int bm, int bn, int bk);
bool gemm_bf16_vec_fits(int bm, int bk, long long N, long long K);
bool gemm_bf16_lds_eligible(int bm, int bn, int bk, long long N, long long K);
bool gemm_bf16_pp_eligible(int bm, int bn, int bk, long long N, long long K);
hipError_t launch_gemm_bf16_lds(const GemmParams& p, int bm, int bn, bool out_bf16, bool witness,
                                hipStream_t stream);
bool gemm_fp8_tile_supported(int bm, int bn, int bk);
bool gemm_fp8_eligible(int bm, long long N, long long K);
bool padd_tile_supported(int tr, int tc);
int padd_tiles_per_step(int tr, int tc);

// Launch shape of a kernel instance: threads and dynamic LDS per workgroup,
// and how many such workgroups one CU holds at once (registers, LDS, waves).
// A persistent launch runs one program per resident slot: CUs x occupancy.
struct KernelInfo {
  int threads;
  int lds_bytes;
  int occupancy;
};
hipError_t launch_gemm_bf16_lds_sk(const GemmParams& p, int bm, int bn, bool out_bf16,
                                   hipStream_t stream);
hipError_t launch_gemm_fp8_sk(const GemmParams& p, int bm, int bn, hipStream_t stream);
hipError_t launch_sk_fixup(const SkFixParams& f, int bm, int bn, bool out_bf16, hipStream_t stream);
hipError_t launch_gemm_bf16_lds_grouped(const GemmParams& p, int bm, int bn, bool out_bf16, bool witness,
                                        hipStream_t stream);
KernelInfo info_gemm_bf16_lds_grouped(int bm, int bn, bool out_bf16);
hipError_t launch_gemm_fp8_grouped(const GemmParams& p, int bm, int bn, bool witness, hipStream_t stream);
KernelInfo info_gemm_fp8_grouped(int bm, int bn);
KernelInfo info_gemm_bf16(int bm, int bn, int bk, bool out_bf16, bool vec);
KernelInfo info_gemm_bf16_lds(int bm, int bn, bool out_bf16);
KernelInfo info_gemm_bf16_pp(bool out_bf16);
hipError_t launch_gemm_bf16_pp(const GemmParams& p, bool out_bf16, bool witness, hipStream_t stream);
KernelInfo info_gemm_fp8(int bm, int bn);
KernelInfo info_padd(int tr, int tc, bool vec);

// Resident workgroups per CU of `kern` (at least 1), after raising its
// dynamic-LDS limit to `lds` bytes.
inline int occupancy_of(const void* kern, int threads, int lds) {
  if (lds > 0) (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, (size_t)lds) != hipSuccess || n < 1)
    n = 1;
  return n;
}

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

// Wall clock (constant rate, see hipDeviceAttributeWallClockRate).
__device__ __forceinline__ long long wall_ticks() { return (long long)wall_clock64(); }

// Shader clock cycle counter of the wave (runs at the current engine clock,
// so cycles / wall time is the clock the program actually ran at).
__device__ __forceinline__ long long shader_cycles() { return (long long)__builtin_readcyclecounter(); }

// Placement of the calling wave: HW_ID low half (CU, SH, SE fields) and the
// XCC id in bits 16-19.
__device__ __forceinline__ int hw_placement() {
  const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_REG_HW_ID, 32 bits
  const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // HW_REG_XCC_ID, 4 bits
  return (int)((hw & 0xffffu) | ((xcc & 0xfu) << 16));
}

// Hardware XCC (XCD) the calling wave runs on.
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xfu);  // HW_REG_XCC_ID, 4 bits
}

// The straggler debug flag: true for the program it slows down (by program
// id, or every program on one hardware XCC).
__device__ __forceinline__ bool is_straggler(const SchedParams& s, int prog) {
  if (s.straggler_program < 0) return false;
  return s.straggler_xcc ? xcc_id() == s.straggler_program : prog == s.straggler_program;
}

// Bounded wait used by the straggler debug flag: returns after `ns`.
__device__ __forceinline__ void spin_ns(int ns, int wall_khz) {
  const long long t0 = wall_ticks();
  const long long ticks = ((long long)ns * wall_khz) / 1000000LL;
  while (wall_ticks() - t0 < ticks) __builtin_amdgcn_s_sleep(2);
}

// Memory operations of the work-stealing claim (pgs::ws_claim) on the
// counters, relaxed device-scope atomics.  ThreadOps: called by the one
// thread that claims for its workgroup.  WaveOps: called by a whole wave with
// every lane active; lane 0 performs the operation and the result is
// broadcast, so the claim's state stays uniform (scalar registers).
struct ThreadOps {
  int* counters;
  int* made = nullptr;  // witness launches: claims per counter (kMaxStealCounters), counted by the claiming thread
  __device__ __forceinline__ int fetch_add(int c, int v) {
    if (made && c < kMaxStealCounters) made[c] += 1;
    return __hip_atomic_fetch_add(counters + c * kCounterStride, v, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ int load(int c) {
    return __hip_atomic_load(counters + c * kCounterStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void store(int c, int v) {
    __hip_atomic_store(counters + c * kCounterStride, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

struct WaveOps {
  int* counters;
  int* made = nullptr;  // witness launches: claims per counter, counted by lane 0
  __device__ __forceinline__ int fetch_add(int c, int v) {
    int r = 0;
    if ((threadIdx.x & 63) == 0) {
      if (made && c < kMaxStealCounters) made[c] += 1;
      r = __hip_atomic_fetch_add(counters + c * kCounterStride, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return __builtin_amdgcn_readfirstlane(r);
  }
  __device__ __forceinline__ int load(int c) {
    int r = 0;
    if ((threadIdx.x & 63) == 0)
      r = __hip_atomic_load(counters + c * kCounterStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(r);
  }
  __device__ __forceinline__ void store(int c, int v) {
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_store(counters + c * kCounterStride, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Per-program view of the scheduler.  Static kinds walk arithmetically.
// Work stealing claims from counter p mod X; work stealing across XCDs starts
// on the counter of the XCD the program runs on and moves on to the others
// as pgs::ws_claim describes.  first()/next() return a tile id or -1 when the
// program is done; for the work-stealing kinds each call may claim, so only
// one thread of the workgroup may call them (or, with first_wave()/
// next_wave(), one whole wave).
struct Walker {
  SchedParams s;
  int p;
  int end;         // static: end of the walk
  pgs::WsWalk ws;  // work stealing: the walk over the counters
  int reset_at;    // per-XCD work stealing with self_reset: see pgs::ws_claim
  int* claim_row = nullptr;  // witness launches: this program's claims per counter

  __device__ __forceinline__ int nx() const { return s.X > 0 ? s.X : 1; }

  __device__ __forceinline__ Walker(const SchedParams& sp, int prog) : s(sp), p(prog) {
    end = 0;
    const int X = nx();
    pgs::ws_start(ws, sp.kind == pgs::kWorkStealingXcc ? xcc_id() % X : prog % X, sp.T, X);
    reset_at = (sp.self_reset && sp.kind == pgs::kWorkStealing)
                   ? pgs::ws_last_claim_value(ws.n, sp.chunk, sp.G, X, ws.x)
                   : -1;
  }

  template <class Ops>
  __device__ __forceinline__ int claim_with(Ops ops) {
    return pgs::ws_claim(ws, s.kind == pgs::kWorkStealingXcc, s.T, s.G, nx(), s.chunk, ops, reset_at);
  }

  // One claim (s.chunk tiles, or a pair / single under paired claims);
  // returns the first claimed id or -1, and sets ws.cend to the claim's end.
  __device__ __forceinline__ int claim() { return claim_with(ThreadOps{s.counters, claim_row}); }

  // End (exclusive) of the claim that starts at tile v (any thread may call it).
  __device__ __forceinline__ int claim_end(int v) const { return pgs::ws_claim_end(v, s.chunk, s.T, nx()); }

  __device__ __forceinline__ int first() {
    if (pgs::work_stealing(s.kind)) return claim();
    return first_static();
  }

  // Static kinds only (no claim code): callers that walk many tiles per
  // step keep the work-stealing path out of their unrolled loops.
  __device__ __forceinline__ int first_static() {
    int v;
    pgs::static_first(s.kind, p, s.T, s.G, v, end);
    return v < end ? v : -1;
  }

  __device__ __forceinline__ int next_static(int v) {
    const int nv = pgs::static_next(s.kind, v, s.G, end);
    return nv < end ? nv : -1;
  }

  // The tile after v: the next one of the current claim, else a new claim.
  __device__ __forceinline__ int next(int v) {
    if (pgs::work_stealing(s.kind)) return v + 1 < ws.cend ? v + 1 : claim();
    return next_static(v);
  }

  // first() / next() called by every lane of one wave (the result and the
  // walk's state are the same in every lane).
  __device__ __forceinline__ int first_wave() {
    if (pgs::work_stealing(s.kind)) return claim_with(WaveOps{s.counters, claim_row});
    return first_static();
  }
  __device__ __forceinline__ int next_wave(int v) {
    if (pgs::work_stealing(s.kind)) return v + 1 < ws.cend ? v + 1 : claim_with(WaveOps{s.counters, claim_row});
    return next_static(v);
  }

  __device__ __forceinline__ void tile_coords(int v, int& pid_m, int& pid_n) const {
    pgs::decode(s.kind, v, s.num_pid_m, s.num_pid_n, s.gs, pid_m, pid_n);
  }
};

#endif

}  // namespace pgk
