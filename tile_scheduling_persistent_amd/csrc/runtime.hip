// C ABI of the library (include/pgemm.h): configuration, argument checks,
// stream-ordered counter reset and kernel launch.
//
// The configuration object follows the matmul wrapper reviewed in "Work
// Stealing Scheduler Kernel" (tritonBLAS PR #65): it reads the CU count of
// the device once, preallocates the int32 per-XCD tile counters (max_xcds
// entries, 16 by default) for reuse across calls, and the counters are reset
// before every work-stealing launch.  The reviewed defects become checks
// here: the device is an int ordinal; the XCD count may not exceed the
// counter array; only device pointers are accepted.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/pgemm.h"
#include "common.hpp"

// A program numbering choose_order made, by the scheduler parameters, the
// tile and (several problems per launch) each problem's first tile id and
// tile grid.
static_assert(PGEMM_MAX_PROBLEMS == pgk::kMaxGemmProblems, "header states the problem limit");
constexpr int kOrderKey = 10 + 3 * pgk::kMaxGemmProblems;
constexpr int kOrderCache = 8;
struct OrderChoice {
  bool valid = false;
  int key[kOrderKey];
  int xcd_major;
};

struct pgemm_config {
  int device;
  int num_cus;
  int num_xcds;
  int capacity;
  int wall_khz;
  int clock_khz;
  int lds_per_cu;
  char arch[64];
  int* counters;  // device, [capacity * pgk::kCounterStride]; counter x at x * kCounterStride
  bool counters_dirty;  // the counters may hold a launch's values (see reset_counters)
  float* ws;          // stream-K partial-sum workspace (device), grown on demand
  size_t ws_bytes;
  unsigned char* scratch;  // this device's address of the static `scratch` array
  OrderChoice order_choice[kOrderCache];  // recent numbering decisions (choose_order)
  int order_next = 0;                     // slot the next new decision replaces
  // witness buffers (device)
  int64_t w_tiles;
  int w_programs;
  int* w_visits;
  int* w_owner;
  int* w_order;
  long long* w_t_start;
  long long* w_t_end;
  long long* w_cycles;
  int* w_hw_id;
  int* w_n_tiles;
  int* w_claims;  // [w_programs][kMaxStealCounters]
};

namespace {

constexpr int kDefaultMaxXcds = 16;
constexpr int kDefaultGroup = 8;     // GEMM: rows of tiles per group of the grouped order
// The add: one row of tiles per group, so the grouped order (and the ranges
// of work stealing) walk the tiles in memory order.  Grouping rows keeps
// operand panels in L2 for a GEMM; an add reuses nothing, and tiles taken
// side by side from one row spread over the memory channels, where a group
// of rows walked column by column puts the tiles in flight in a few narrow
// column bands (measured at 8192x8192: work stealing 5.6 -> 6.1 TB/s at
// 128x128 tiles, 4.2 -> 4.8 at 32x16).
constexpr int kDefaultAddGroup = 1;
constexpr int kMaxGemmChunk = 64;  // tiles per work-stealing claim, GEMM
// PGEMM_PIPELINE_DEFAULT takes the ping-pong kernel where it applies.
constexpr bool kPingPongDefault = false;

pgemm_status from_hip(hipError_t e) {
  if (e == hipSuccess) return PGEMM_OK;
  if (e == hipErrorOutOfMemory) return PGEMM_ERR_OOM;
  return PGEMM_ERR_DEVICE;
}

// Is p a device (or managed) allocation of device `dev`?
bool is_device_ptr(const void* p, int dev) {
  if (p == nullptr) return false;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return false;
  return attr.device == dev;
}

// Does [p, p + bytes) lie inside one device allocation of device `dev`?  The
// kernels take their address ranges from the sizes of the call, not from the
// allocation, so a buffer shorter than the sizes say would be read or written
// past its end.
bool device_range(const void* p, size_t bytes, int dev) {
  if (!is_device_ptr(p, dev)) return false;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  const uintptr_t b = (uintptr_t)base, q = (uintptr_t)p;
  return q >= b && q - b <= size && bytes <= size - (q - b);
}

// M * N * element size, or SIZE_MAX if it does not fit (then no allocation holds it).
size_t span_bytes(int64_t rows, int64_t cols, size_t esz) {
  if (rows <= 0 || cols <= 0) return 0;
  const unsigned __int128 b = (unsigned __int128)rows * (unsigned __int128)cols * esz;
  return b > (unsigned __int128)SIZE_MAX ? SIZE_MAX : (size_t)b;
}

bool validate_only(const pgemm_args* args) {
  return args && (args->debug_flags & PGEMM_DEBUG_VALIDATE_ONLY);
}

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(dev) == hipSuccess) ok = true;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

void free_witness(pgemm_config* c) {
  void* ptrs[] = {c->w_visits, c->w_owner, c->w_order, c->w_t_start,
                  c->w_t_end, c->w_cycles, c->w_hw_id, c->w_n_tiles, c->w_claims};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  c->w_visits = c->w_owner = c->w_order = c->w_hw_id = c->w_n_tiles = c->w_claims = nullptr;
  c->w_t_start = c->w_t_end = c->w_cycles = nullptr;
  c->w_tiles = 0;
  c->w_programs = 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Common scheduler setup; returns PGEMM_OK or an error (nothing enqueued).
// balance: GEMM (balanced default grid, group size 8); the add keeps the full
// grid and takes group size 1 by default.  The
// program numbering starts as the workgroup order; GEMM paths then call
// choose_order.
pgemm_status make_sched(pgemm_config* cfg, pgemm_sched sched, const pgemm_args* args,
                        int num_pid_m, int num_pid_n, int default_grid, bool balance,
                        pgk::SchedParams& s) {
  const int default_group = balance ? kDefaultGroup : kDefaultAddGroup;
  if ((int)sched < 0 || (int)sched > 6) return PGEMM_ERR_INVALID;
  const int64_t T = (int64_t)num_pid_m * num_pid_n;
  if (T > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  s.kind = (int)sched;
  s.T = (int)T;
  s.G = (args && args->grid) ? args->grid : default_grid;
  s.X = cfg->num_xcds;
  // GEMM default: trimmed to the balanced grid (stream-K keeps every
  // program: it splits the last round's tiles over all of them).
  if (balance && !(args && args->grid) && sched != PGEMM_SCHED_STREAM_K)
    s.G = pgs::balanced_grid(s.T, s.G, s.X);
  s.gs = (args && args->group_size) ? args->group_size : default_group;
  s.num_pid_m = num_pid_m;
  s.num_pid_n = num_pid_n;
  s.counters = cfg->counters;
  s.self_reset = 0;
  s.chunk = 1;
  if (args && args->claim_chunk) {
    if (args->claim_chunk == PGEMM_CLAIM_PAIRS)
      s.chunk = -1;
    else if (args->claim_chunk < 1 || args->claim_chunk > kMaxGemmChunk)
      return PGEMM_ERR_INVALID;
    else
      s.chunk = args->claim_chunk;
  }
  s.straggler_program = -1;
  s.straggler_ns = 0;
  s.straggler_xcc = 0;
  s.wall_khz = cfg->wall_khz;
  if (s.G < 1 || s.gs < 1) return PGEMM_ERR_INVALID;
  const int order = args ? args->program_order : PGEMM_ORDER_DEFAULT;
  if (order != PGEMM_ORDER_DEFAULT && order != PGEMM_ORDER_DISPATCH && order != PGEMM_ORDER_XCD_MAJOR)
    return PGEMM_ERR_INVALID;
  s.xcd_major = 0;
  if (s.kind == pgs::kWorkStealing && s.G < s.X) return PGEMM_ERR_INVALID;
  if (s.kind == pgs::kWorkStealingXcc && s.X > pgk::kMaxStealCounters) return PGEMM_ERR_UNSUPPORTED;
  if (s.X < 1 || s.X > cfg->capacity) return PGEMM_ERR_INVALID;
  if (args && (args->debug_flags & PGEMM_DEBUG_STRAGGLER)) {
    if (args->straggler_ns < 0 || args->straggler_ns > 1000000000) return PGEMM_ERR_INVALID;
    s.straggler_program = args->straggler_program;
    s.straggler_ns = args->straggler_ns;
  }
  if (args && (args->debug_flags & PGEMM_DEBUG_STRAGGLER_XCC)) {
    if (args->debug_flags & PGEMM_DEBUG_STRAGGLER) return PGEMM_ERR_INVALID;
    if (args->straggler_ns < 0 || args->straggler_ns > 1000000000) return PGEMM_ERR_INVALID;
    s.straggler_program = args->straggler_program;
    s.straggler_ns = args->straggler_ns;
    s.straggler_xcc = 1;
  }
  return PGEMM_OK;
}

// Operand panels the first tiles of a static walk's programs touch, summed
// over the XCDs (the workgroups of one XCD are one residue class of i mod X):
// distinct rows of tiles
// weighted by the tile's rows (bm) plus distinct columns of tiles weighted by
// its columns (bn), per problem.  Proportional to the bytes each XCD's L2
// has to fetch for its programs' first round.  gp / ngemm: the problems of a
// grouped launch (virtual tile ids), or none for one GEMM.
int64_t first_round_panels(const pgk::SchedParams& s, int xcd_major, int bm, int bn,
                           const pgk::GemmProblem* gp, int ngemm) {
  std::vector<std::vector<int64_t>> rows(s.X), cols(s.X);
  for (int hw = 0; hw < s.G; ++hw) {
    const int q = pgs::program_of(hw, s.G, s.X, xcd_major);
    int v, end;
    pgs::static_first(s.kind, q, s.T, s.G, v, end);
    if (v >= end) continue;
    int g = 0, local = v, npm = s.num_pid_m, npn = s.num_pid_n;
    for (int i = 1; i < ngemm; ++i)
      if (v >= gp[i].tile0) g = i;
    if (ngemm > 0) {
      local = v - gp[g].tile0;
      npm = gp[g].npm;
      npn = gp[g].npn;
    }
    int pm, pn;
    pgs::decode(s.kind, local, npm, npn, s.gs, pm, pn);
    rows[hw % s.X].push_back(((int64_t)g << 32) | (uint32_t)pm);
    cols[hw % s.X].push_back(((int64_t)g << 32) | (uint32_t)pn);
  }
  int64_t total = 0;
  for (int x = 0; x < s.X; ++x) {
    for (auto* k : {&rows[x], &cols[x]}) {
      std::sort(k->begin(), k->end());
      const int64_t n = std::unique(k->begin(), k->end()) - k->begin();
      total += n * (k == &rows[x] ? bm : bn);
    }
  }
  return total;
}

// Program numbering of a GEMM's static walk (pgemm_args.program_order).
// DEFAULT takes XCD-major numbering where it makes the first round touch
// fewer operand panels per XCD than the workgroup order, which depends on
// the decode: for the grouped order, an XCD's consecutive ids form a compact
// block of tiles; for the plain decode with many rows of tiles, they form a
// column, and the round robin of the workgroup order is the compact one.
void choose_order(pgemm_config* cfg, const pgemm_args* args, pgk::SchedParams& s, int bm, int bn,
                  const pgk::GemmProblem* gp, int ngemm) {
  s.xcd_major = 0;
  const int order = args ? args->program_order : PGEMM_ORDER_DEFAULT;
  if (order == PGEMM_ORDER_DISPATCH || pgs::work_stealing(s.kind) || s.kind == pgs::kStreamK ||
      s.X < 2 || s.G % s.X != 0)
    return;
  if (order == PGEMM_ORDER_XCD_MAJOR) {
    s.xcd_major = 1;
    return;
  }
  int key[kOrderKey] = {s.kind, s.T, s.G, s.X, s.gs, s.num_pid_m, s.num_pid_n, bm, bn, ngemm};
  for (int g = 0; g < ngemm; ++g) {
    key[10 + 3 * g] = gp[g].tile0;
    key[11 + 3 * g] = gp[g].npm;
    key[12 + 3 * g] = gp[g].npn;
  }
  for (const OrderChoice& c : cfg->order_choice)
    if (c.valid && memcmp(c.key, key, sizeof(key)) == 0) {
      s.xcd_major = c.xcd_major;
      return;
    }
  s.xcd_major = first_round_panels(s, 1, bm, bn, gp, ngemm) < first_round_panels(s, 0, bm, bn, gp, ngemm);
  OrderChoice& c = cfg->order_choice[cfg->order_next];
  cfg->order_next = (cfg->order_next + 1) % kOrderCache;
  memcpy(c.key, key, sizeof(key));
  c.xcd_major = s.xcd_major;
  c.valid = true;
}

// Kernel a GEMM call takes, from shapes, formats, tile and pointer alignment
// (pointers may be null: taken as 16-byte aligned).
struct GemmChoice {
  int bm, bn, bk;
  pgemm_kernel kernel;
  bool out_bf16;
  bool vec;  // register-staged kernel: 16-byte vector path
};

pgemm_status choose_gemm(int64_t M, int64_t N, int64_t K, pgemm_dtype dtype, pgemm_sched sched,
                         const pgemm_args* args, const void* A, const void* B, const void* C, GemmChoice& ch) {
  if (M < 1 || N < 1 || K < 1 || M > 0x7fffffffLL || N > 0x7fffffffLL || K > 0x7fffffffLL)
    return PGEMM_ERR_INVALID;
  const bool fp8 = dtype == PGEMM_FP8E4M3_B128_OUT_BF16;
  if (!fp8 && dtype != PGEMM_BF16_OUT_F32 && dtype != PGEMM_BF16_OUT_BF16)
    return PGEMM_ERR_INVALID;
  ch.bm = 256;
  ch.bn = 256;
  ch.bk = fp8 ? 128 : 64;
  if (args && (args->tile_m || args->tile_n || args->tile_k)) {
    ch.bm = args->tile_m;
    ch.bn = args->tile_n;
    ch.bk = args->tile_k;
  }
  if (ch.bm < 1 || ch.bn < 1 || ch.bk < 1) return PGEMM_ERR_INVALID;
  ch.out_bf16 = dtype != PGEMM_BF16_OUT_F32;
  ch.vec = false;
  const bool al = (!A || aligned(A, 16)) && (!B || aligned(B, 16)) && (!C || aligned(C, 16));
  if (fp8) {
    if (K % 128 != 0) return PGEMM_ERR_INVALID;
    if (!pgk::gemm_fp8_tile_supported(ch.bm, ch.bn, ch.bk)) return PGEMM_ERR_UNSUPPORTED;
    // the fp8 kernel moves 16-byte chunks of B rows and of C
    if (!pgk::gemm_fp8_eligible(ch.bm, N, K) || !al) return PGEMM_ERR_UNSUPPORTED;
    ch.kernel = PGEMM_KERNEL_FP8;
    return PGEMM_OK;
  }
  if (!pgk::gemm_bf16_tile_supported(ch.bm, ch.bn, ch.bk)) return PGEMM_ERR_UNSUPPORTED;
  const bool staged = args && (args->debug_flags & PGEMM_DEBUG_REGISTER_STAGED);
  const int pipe = args ? args->pipeline : PGEMM_PIPELINE_DEFAULT;
  if (pipe < PGEMM_PIPELINE_DEFAULT || pipe > PGEMM_PIPELINE_PINGPONG) return PGEMM_ERR_INVALID;
  if (!staged && al && pgk::gemm_bf16_lds_eligible(ch.bm, ch.bn, ch.bk, N, K)) {
    ch.kernel = PGEMM_KERNEL_BF16_LDS;
    // the ping-pong kernel: 256x256x64 tiles, one problem, not stream-K
    const bool pp = sched != PGEMM_SCHED_STREAM_K && pgk::gemm_bf16_pp_eligible(ch.bm, ch.bn, ch.bk, N, K);
    if (pipe == PGEMM_PIPELINE_PINGPONG && !pp) return PGEMM_ERR_UNSUPPORTED;
    if (pipe == PGEMM_PIPELINE_PINGPONG || (pipe == PGEMM_PIPELINE_DEFAULT && pp && kPingPongDefault))
      ch.kernel = PGEMM_KERNEL_BF16_PINGPONG;
  } else if (pipe == PGEMM_PIPELINE_PINGPONG) {
    return PGEMM_ERR_UNSUPPORTED;
  } else {
    ch.kernel = PGEMM_KERNEL_BF16_STAGED;
    ch.vec = (K % 8 == 0) && (N % 8 == 0) && al && pgk::gemm_bf16_vec_fits(ch.bm, ch.bk, N, K);
  }
  return PGEMM_OK;
}

pgk::KernelInfo gemm_info(const GemmChoice& ch) {
  switch (ch.kernel) {
    case PGEMM_KERNEL_FP8: return pgk::info_gemm_fp8(ch.bm, ch.bn);
    case PGEMM_KERNEL_BF16_LDS: return pgk::info_gemm_bf16_lds(ch.bm, ch.bn, ch.out_bf16);
    case PGEMM_KERNEL_BF16_PINGPONG: return pgk::info_gemm_bf16_pp(ch.out_bf16);
    default: return pgk::info_gemm_bf16(ch.bm, ch.bn, ch.bk, ch.out_bf16, ch.vec);
  }
}

void fill_plan(const pgk::SchedParams& s, const pgk::KernelInfo& ki, int bm, int bn, int bk,
               pgemm_kernel kernel, pgemm_plan* out) {
  out->grid = s.G;
  out->occupancy = ki.occupancy;
  out->tiles = s.T;
  out->tile_m = bm;
  out->tile_n = bn;
  out->tile_k = bk;
  out->threads = ki.threads;
  out->lds_bytes = ki.lds_bytes;
  out->kernel = kernel;
  out->xcd_major = s.xcd_major;
}

pgemm_status make_witness(pgemm_config* cfg, const pgemm_args* args, const pgk::SchedParams& s,
                          pgk::Witness& w, bool& on, hipStream_t stream) {
  memset(&w, 0, sizeof(w));
  on = args && (args->debug_flags & PGEMM_DEBUG_WITNESS);
  if (!on) return PGEMM_OK;
  if (cfg->w_visits == nullptr || s.T > cfg->w_tiles || s.G > cfg->w_programs)
    return PGEMM_ERR_INVALID;
  w.visits = cfg->w_visits;
  w.owner = cfg->w_owner;
  w.order = cfg->w_order;
  w.t_start = cfg->w_t_start;
  w.t_end = cfg->w_t_end;
  w.cycles = cfg->w_cycles;
  w.hw_id = cfg->w_hw_id;
  w.n_tiles = cfg->w_n_tiles;
  w.claims = cfg->w_claims;
  // visits and claims start at 0, owner / order at -1 (fill kernels, no memset nodes)
  hipError_t e = pgk::launch_fill_i32(w.visits, s.T, 0, stream);
  if (e == hipSuccess) e = pgk::launch_fill_i32(w.claims, s.G * pgk::kMaxStealCounters, 0, stream);
  if (e == hipSuccess) e = pgk::launch_fill_i32(w.owner, s.T, -1, stream);
  if (e == hipSuccess) e = pgk::launch_fill_i32(w.order, s.T, -1, stream);
  if (e == hipSuccess) e = pgk::launch_fill_i32(w.n_tiles, s.G, 0, stream);
  return e == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH;
}

// Work-stealing counters before a launch.  Per-XCD work stealing leaves its
// counters zeroed at the end of the launch (the last failing claim on each
// zeroes it, pgs::ws_claim), so the stream-ordered fill kernel the pages'
// reset-before-every-launch calls for runs only when the counters may hold
// values of an earlier launch: after a witness launch (its final counters are
// read back), after stealing across XCDs (whose failing claims per counter
// vary), after a launch that skipped the reset, and on first use.  `dirty`
// tracks that for one counter array of n_counters entries.
pgemm_status reset_counters(const pgemm_args* args, pgk::SchedParams& s, int n_counters, bool* dirty,
                            bool witness, hipStream_t stream) {
  s.self_reset = 0;
  if (!pgs::work_stealing(s.kind)) return PGEMM_OK;
  const bool skip = args && (args->debug_flags & PGEMM_DEBUG_SKIP_RESET);
  const bool self = s.kind == pgs::kWorkStealing && !witness && !skip;
  if (!skip && (*dirty || !self)) {
    // a fill kernel rather than a memset node, so that the call may be captured
    if (pgk::launch_zero_i32(s.counters, n_counters * pgk::kCounterStride, stream) != hipSuccess)
      return PGEMM_ERR_LAUNCH;
  }
  s.self_reset = self ? 1 : 0;
  *dirty = !self;
  return PGEMM_OK;
}


// Stream-K workspace of at least `bytes`: two partial-sum slots per program.
// The config allocates it for the default grid of every stream-K tile when
// it is created, so only a call with a larger grid (args->grid) lands here:
// the workspace then grows with hipFree / hipMalloc after synchronising the
// device, so no launch still uses the old buffer.  Under stream capture a
// synchronisation is not allowed: PGEMM_ERR_INVALID, nothing enqueued.
pgemm_status ensure_workspace(pgemm_config* cfg, size_t bytes, hipStream_t stream) {
  if (cfg->ws_bytes >= bytes) return PGEMM_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return PGEMM_ERR_DEVICE;
  if (cap != hipStreamCaptureStatusNone) return PGEMM_ERR_INVALID;
  if (cfg->ws) {
    if (hipDeviceSynchronize() != hipSuccess) return PGEMM_ERR_DEVICE;
    (void)hipFree(cfg->ws);
    cfg->ws = nullptr;
    cfg->ws_bytes = 0;
  }
  if (hipMalloc((void**)&cfg->ws, bytes) != hipSuccess) {
    cfg->ws = nullptr;
    return PGEMM_ERR_OOM;
  }
  cfg->ws_bytes = bytes;
  return PGEMM_OK;
}

// Device memory of the allocation-free entry point (pgemm_run_noalloc): one
// static array per device, `scratch`, holding the work-stealing counters
// (kScratchCounters blocks of 256 bytes) followed by the stream-K partial-sum
// slots.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol): pgemm_config_create looks up the
// device address with hipGetSymbolAddress, once per device with that device
// current, and every use goes through that address.  Every call on a GPU
// shares its array; calls that overlap on one GPU race.
constexpr int kScratchCounters = 16;
constexpr size_t kScratchCounterBytes = (size_t)kScratchCounters * pgk::kCounterStride * sizeof(int);
constexpr size_t kScratchWsBytes = (size_t)64 << 20;
constexpr size_t kScratchBytes = kScratchCounterBytes + kScratchWsBytes;
static_assert(kScratchCounterBytes % 256 == 0, "partial sums start 256-byte aligned");
static_assert(PGEMM_NOALLOC_SCRATCH_BYTES == kScratchBytes, "header states the scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices];  // per device: address of `scratch` there, or null
bool g_scratch_dirty[kMaxDevices] = {true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true,
                                     true, true, true, true, true, true, true, true};  // first use fills

// Address of `scratch` on `device` (the caller has made it current).
pgemm_status scratch_address(int device, unsigned char** out) {
  if (device < 0 || device >= kMaxDevices) return PGEMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[device]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return PGEMM_ERR_DEVICE;
    }
    g_scratch[device] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch[device];
  return PGEMM_OK;
}

// Device scratch of one GEMM call: the work-stealing counters and the
// stream-K partial sums, either the config's allocations (which may grow for
// a larger grid) or the static scratch (which never does).
struct CallBuffers {
  int* counters;
  int n_counters;
  bool* dirty;  // the counters may hold a launch's values
  float* ws;
  size_t ws_bytes;
  bool growable;
};

pgemm_status gemm_call(pgemm_config* cfg, const void* A, const void* B, void* C, int64_t M, int64_t N,
                       int64_t K, pgemm_dtype dtype, pgemm_sched sched, const pgemm_args* args,
                       void* hip_stream, CallBuffers buf);

}  // namespace

extern "C" {

const char* pgemm_status_str(pgemm_status s) {
  switch (s) {
    case PGEMM_OK: return "ok";
    case PGEMM_ERR_INVALID: return "invalid argument";
    case PGEMM_ERR_UNSUPPORTED: return "unsupported device or kernel variant";
    case PGEMM_ERR_DEVICE: return "HIP runtime error";
    case PGEMM_ERR_OOM: return "device out of memory";
    case PGEMM_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

pgemm_status pgemm_config_create(int device, int max_xcds, pgemm_config** out) {
  if (out == nullptr) return PGEMM_ERR_INVALID;
  *out = nullptr;
  if (max_xcds < 0 || max_xcds > 1024) return PGEMM_ERR_INVALID;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return PGEMM_ERR_DEVICE;
  if (device < 0 || device >= ndev) return PGEMM_ERR_INVALID;
  DeviceGuard g(device);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return PGEMM_ERR_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return PGEMM_ERR_UNSUPPORTED;
  int xcc = 0, wall = 0;
  if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, device) != hipSuccess || xcc < 1)
    return PGEMM_ERR_DEVICE;
  if (hipDeviceGetAttribute(&wall, hipDeviceAttributeWallClockRate, device) != hipSuccess)
    wall = 100000;
  const int cap = max_xcds ? max_xcds : kDefaultMaxXcds;
  if (xcc > cap) return PGEMM_ERR_INVALID;

  pgemm_config* c = new (std::nothrow) pgemm_config();
  if (!c) return PGEMM_ERR_OOM;
  memset(c, 0, sizeof(*c));
  c->device = device;
  c->num_cus = prop.multiProcessorCount;
  c->num_xcds = xcc;
  c->capacity = cap;
  c->wall_khz = wall > 0 ? wall : 100000;
  c->clock_khz = prop.clockRate;
  c->lds_per_cu = (int)prop.maxSharedMemoryPerMultiProcessor;
  strncpy(c->arch, prop.gcnArchName, sizeof(c->arch) - 1);
  const size_t cbytes = sizeof(int) * (size_t)cap * pgk::kCounterStride;
  // Stream-K partial sums: two fp32 tile slots per program at the default
  // grid (CUs x resident workgroups) of every tile the stream-K kernels take,
  // allocated once here so that pgemm_run does not allocate.
  size_t wsb = 0;
  {
    const int bf16_tiles[2][2] = {{256, 256}, {128, 128}};
    const int fp8_tiles[3][2] = {{256, 256}, {128, 128}, {128, 256}};
    for (const auto& t : bf16_tiles) {
      const pgk::KernelInfo ki = pgk::info_gemm_bf16_lds(t[0], t[1], true);
      const size_t b = (size_t)c->num_cus * (size_t)ki.occupancy * 2 * (size_t)t[0] * t[1] * sizeof(float);
      wsb = b > wsb ? b : wsb;
    }
    for (const auto& t : fp8_tiles) {
      const pgk::KernelInfo ki = pgk::info_gemm_fp8(t[0], t[1]);
      const size_t b = (size_t)c->num_cus * (size_t)ki.occupancy * 2 * (size_t)t[0] * t[1] * sizeof(float);
      wsb = b > wsb ? b : wsb;
    }
  }
  if (scratch_address(device, &c->scratch) != PGEMM_OK) {
    delete c;
    return PGEMM_ERR_DEVICE;
  }
  hipError_t e = hipMalloc((void**)&c->counters, cbytes);
  if (e == hipSuccess) e = hipMemset(c->counters, 0, cbytes);
  if (e == hipSuccess) e = hipMalloc((void**)&c->ws, wsb);
  if (e == hipSuccess) c->ws_bytes = wsb;
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    if (c->counters) (void)hipFree(c->counters);
    if (c->ws) (void)hipFree(c->ws);
    delete c;
    return from_hip(e);
  }
  *out = c;
  return PGEMM_OK;
}

pgemm_status pgemm_config_query(const pgemm_config* cfg, pgemm_info* info) {
  if (!cfg || !info) return PGEMM_ERR_INVALID;
  memset(info, 0, sizeof(*info));
  info->num_cus = cfg->num_cus;
  info->num_xcds = cfg->num_xcds;
  info->counter_capacity = cfg->capacity;
  info->wall_clock_khz = cfg->wall_khz;
  info->clock_khz = cfg->clock_khz;
  info->lds_bytes_per_cu = cfg->lds_per_cu;
  strncpy(info->arch, cfg->arch, sizeof(info->arch) - 1);
  return PGEMM_OK;
}

pgemm_status pgemm_config_destroy(pgemm_config* cfg) {
  if (!cfg) return PGEMM_OK;
  DeviceGuard g(cfg->device);
  free_witness(cfg);
  if (cfg->counters) (void)hipFree(cfg->counters);
  if (cfg->ws) (void)hipFree(cfg->ws);
  delete cfg;
  return PGEMM_OK;
}

static bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  return an > 0 && bn > 0 && x < y + bn && y < x + an;
}

pgemm_status padd_run_multi(pgemm_config* cfg, const padd_problem* problems, int count,
                            int tile_rows, int tile_cols, pgemm_sched sched,
                            const pgemm_args* args, void* hip_stream) {
  if (!cfg || !problems || count < 1 || count > PADD_MAX_PROBLEMS) return PGEMM_ERR_INVALID;
  if (tile_rows < 1 || tile_cols < 1) return PGEMM_ERR_INVALID;
  if (!pgk::padd_tile_supported(tile_rows, tile_cols)) return PGEMM_ERR_UNSUPPORTED;
  if (args && args->claim_chunk == PGEMM_CLAIM_PAIRS) return PGEMM_ERR_UNSUPPORTED;
  const int dev = cfg->device;
  pgk::AddParams p;
  memset(&p, 0, sizeof(p));
  p.nprob = count;
  int64_t total = 0;
  bool vec = true;
  for (int g = 0; g < count; ++g) {
    const padd_problem& q = problems[g];
    if (!q.X || !q.Y || !q.C) return PGEMM_ERR_INVALID;
    if (q.rows < 0 || q.cols < 0 || q.rows > 0x7fffffffLL || q.cols > 0x7fffffffLL) return PGEMM_ERR_INVALID;
    const size_t bytes = span_bytes(q.rows, q.cols, 4);
    if (!device_range(q.X, bytes, dev) || !device_range(q.Y, bytes, dev) || !device_range(q.C, bytes, dev))
      return PGEMM_ERR_INVALID;
    // C against every buffer: its own X / Y may be the same buffer, nothing else may touch it
    for (int h = 0; h < count; ++h) {
      const padd_problem& o = problems[h];
      const size_t ob = (size_t)o.rows * (size_t)o.cols * 4;
      const void* bufs[3] = {o.X, o.Y, o.C};
      for (int b = 0; b < 3; ++b) {
        if (h == g && b == 2) continue;
        const bool same = h == g && bufs[b] == (const void*)q.C;
        if (!same && overlaps(q.C, bytes, bufs[b], ob)) return PGEMM_ERR_INVALID;
      }
    }
    const int64_t npm = (q.rows + tile_rows - 1) / tile_rows, npn = (q.cols + tile_cols - 1) / tile_cols;
    pgk::AddProblem& a = p.prob[g];
    a.X = q.X;
    a.Y = q.Y;
    a.C = q.C;
    a.rows = (int)q.rows;
    a.cols = (int)q.cols;
    a.tile0 = (int)total;
    a.npm = (int)npm;
    a.npn = (int)npn;
    total += npm * npn;
    if (total > 0x7fffffffLL) return PGEMM_ERR_INVALID;
    if (q.rows > 0 && q.cols > 0)
      vec = vec && (q.cols % 4 == 0) && aligned(q.X, 16) && aligned(q.Y, 16) && aligned(q.C, 16);
  }
  if (total == 0) return PGEMM_OK;  // nothing to do
  p.X = p.prob[0].X;
  p.Y = p.prob[0].Y;
  p.C = p.prob[0].C;
  DeviceGuard gd(dev);
  if (!gd.ok) return PGEMM_ERR_DEVICE;
  const pgk::KernelInfo ki = pgk::info_padd(tile_rows, tile_cols, vec);
  pgemm_status st = make_sched(cfg, sched, args, (int)total, 1, cfg->num_cus * ki.occupancy, false, p.s);
  if (st != PGEMM_OK) return st;
  const int step = pgk::padd_tiles_per_step(tile_rows, tile_cols);
  p.s.chunk = step;
  if (args && args->claim_chunk) {
    if (args->claim_chunk < 1 || args->claim_chunk > step) return PGEMM_ERR_INVALID;
    p.s.chunk = args->claim_chunk;
  }
  if (validate_only(args)) return PGEMM_OK;
  hipStream_t stream = (hipStream_t)hip_stream;
  bool witness = false;
  st = make_witness(cfg, args, p.s, p.w, witness, stream);
  if (st != PGEMM_OK) return st;
  st = reset_counters(args, p.s, cfg->capacity, &cfg->counters_dirty, witness, stream);
  if (st != PGEMM_OK) return st;
  hipError_t e = pgk::launch_padd_multi(p, tile_rows, tile_cols, vec, witness, stream);
  if (e == hipErrorInvalidValue) return PGEMM_ERR_UNSUPPORTED;
  return e == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH;
}

pgemm_status pgemm_run_grouped(pgemm_config* cfg, const pgemm_problem* problems, int count,
                               pgemm_dtype dtype, pgemm_sched sched, const pgemm_args* args,
                               void* hip_stream) {
  if (!cfg || !problems || count < 1 || count > PGEMM_MAX_PROBLEMS) return PGEMM_ERR_INVALID;
  const bool fp8 = dtype == PGEMM_FP8E4M3_B128_OUT_BF16;
  if (!fp8 && dtype != PGEMM_BF16_OUT_F32 && dtype != PGEMM_BF16_OUT_BF16) return PGEMM_ERR_INVALID;
  if ((int)sched == PGEMM_SCHED_STREAM_K) return PGEMM_ERR_UNSUPPORTED;
  if (args && (args->debug_flags & PGEMM_DEBUG_REGISTER_STAGED)) return PGEMM_ERR_UNSUPPORTED;
  if (args && args->pipeline == PGEMM_PIPELINE_PINGPONG) return PGEMM_ERR_UNSUPPORTED;  // four-wave kernel only
  if (args && (args->pipeline < PGEMM_PIPELINE_DEFAULT || args->pipeline > PGEMM_PIPELINE_PINGPONG))
    return PGEMM_ERR_INVALID;
  int bm = 256, bn = 256, bk = fp8 ? 128 : 64;
  if (args && (args->tile_m || args->tile_n || args->tile_k)) {
    bm = args->tile_m;
    bn = args->tile_n;
    bk = args->tile_k;
  }
  if (bm < 1 || bn < 1 || bk < 1) return PGEMM_ERR_INVALID;
  const int dev = cfg->device;
  const size_t csz = dtype == PGEMM_BF16_OUT_F32 ? 4 : 2;
  pgk::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.ngemm = count;
  int64_t total = 0;
  for (int g = 0; g < count; ++g) {
    const pgemm_problem& q = problems[g];
    if (!q.A || !q.B || !q.C) return PGEMM_ERR_INVALID;
    if (q.M < 0 || q.N < 0 || q.K < 1 || q.M > 0x7fffffffLL || q.N > 0x7fffffffLL || q.K > 0x7fffffffLL)
      return PGEMM_ERR_INVALID;
    const size_t qesz = fp8 ? 1 : 2;
    if (!device_range(q.A, span_bytes(q.M, q.K, qesz), dev) || !device_range(q.B, span_bytes(q.K, q.N, qesz), dev) ||
        !device_range(q.C, span_bytes(q.M, q.N, csz), dev))
      return PGEMM_ERR_INVALID;
    if (fp8) {
      if (!q.a_scale || !q.b_scale || !device_range(q.a_scale, span_bytes(q.K / 128, q.M, 1), dev) ||
          !device_range(q.b_scale, span_bytes(q.K / 128, q.N, 1), dev))
        return PGEMM_ERR_INVALID;
      if (q.K % 128 != 0) return PGEMM_ERR_INVALID;
      if (!aligned(q.A, 16) || !aligned(q.B, 16) || !aligned(q.C, 16) ||
          !pgk::gemm_fp8_tile_supported(bm, bn, bk) || !pgk::gemm_fp8_eligible(bm, q.N, q.K))
        return PGEMM_ERR_UNSUPPORTED;
    } else if (!aligned(q.A, 16) || !aligned(q.B, 16) || !aligned(q.C, 16) ||
               !pgk::gemm_bf16_lds_eligible(bm, bn, bk, q.N, q.K)) {
      return PGEMM_ERR_UNSUPPORTED;
    }
    // each C overlaps no operand and no other output
    const size_t cb = (size_t)q.M * q.N * csz;
    const size_t esz = fp8 ? 1 : 2;
    for (int h = 0; h < count; ++h) {
      const pgemm_problem& o = problems[h];
      if (overlaps(q.C, cb, o.A, (size_t)o.M * o.K * esz) || overlaps(q.C, cb, o.B, (size_t)o.K * o.N * esz))
        return PGEMM_ERR_INVALID;
      if (fp8 && (overlaps(q.C, cb, o.a_scale, (size_t)(o.K / 128) * o.M) ||
                  overlaps(q.C, cb, o.b_scale, (size_t)(o.K / 128) * o.N)))
        return PGEMM_ERR_INVALID;
      if (h != g && overlaps(q.C, cb, o.C, (size_t)o.M * o.N * csz)) return PGEMM_ERR_INVALID;
    }
    const int64_t npm = (q.M + bm - 1) / bm, npn = (q.N + bn - 1) / bn;
    pgk::GemmProblem& a = p.gp[g];
    a.A = q.A;
    a.B = q.B;
    a.C = q.C;
    a.sa = fp8 ? q.a_scale : nullptr;
    a.sb = fp8 ? q.b_scale : nullptr;
    a.M = (int)q.M;
    a.N = (int)q.N;
    a.K = (int)q.K;
    a.tile0 = (int)total;
    a.npm = (int)npm;
    a.npn = (int)npn;
    total += npm * npn;
    if (total > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  }
  if (total == 0) return PGEMM_OK;  // no tiles
  p.A = p.gp[0].A;
  p.B = p.gp[0].B;
  p.C = p.gp[0].C;
  p.sa = p.gp[0].sa;
  p.sb = p.gp[0].sb;
  p.M = p.gp[0].M;
  p.N = p.gp[0].N;
  p.K = p.gp[0].K;
  DeviceGuard gd(dev);
  if (!gd.ok) return PGEMM_ERR_DEVICE;
  const pgk::KernelInfo ki =
      fp8 ? pgk::info_gemm_fp8_grouped(bm, bn) : pgk::info_gemm_bf16_lds_grouped(bm, bn, csz == 2);
  if (ki.threads == 0) return PGEMM_ERR_UNSUPPORTED;
  pgemm_status st = make_sched(cfg, sched, args, (int)total, 1, cfg->num_cus * ki.occupancy, true, p.s);
  if (st != PGEMM_OK) return st;
  choose_order(cfg, args, p.s, bm, bn, p.gp, p.ngemm);
  if (validate_only(args)) return PGEMM_OK;
  hipStream_t stream = (hipStream_t)hip_stream;
  bool witness = false;
  st = make_witness(cfg, args, p.s, p.w, witness, stream);
  if (st != PGEMM_OK) return st;
  st = reset_counters(args, p.s, cfg->capacity, &cfg->counters_dirty, witness, stream);
  if (st != PGEMM_OK) return st;
  hipError_t e = fp8 ? pgk::launch_gemm_fp8_grouped(p, bm, bn, witness, stream)
                     : pgk::launch_gemm_bf16_lds_grouped(p, bm, bn, csz == 2, witness, stream);
  if (e == hipErrorInvalidValue) return PGEMM_ERR_UNSUPPORTED;
  return e == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH;
}

pgemm_status pgemm_witness_enable(pgemm_config* cfg, int64_t max_tiles, int max_programs) {
  if (!cfg || max_tiles < 1 || max_tiles > (1LL << 30) || max_programs < 1 ||
      max_programs > (1 << 20))
    return PGEMM_ERR_INVALID;
  DeviceGuard g(cfg->device);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  if (hipDeviceSynchronize() != hipSuccess) return PGEMM_ERR_DEVICE;
  free_witness(cfg);
  hipError_t e = hipSuccess;
  const size_t t = (size_t)max_tiles, p = (size_t)max_programs;
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_visits, sizeof(int) * t);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_owner, sizeof(int) * t);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_order, sizeof(int) * t);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_t_start, sizeof(long long) * p);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_t_end, sizeof(long long) * p);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_cycles, sizeof(long long) * p);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_hw_id, sizeof(int) * p);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_n_tiles, sizeof(int) * p);
  if (e == hipSuccess) e = hipMalloc((void**)&cfg->w_claims, sizeof(int) * p * pgk::kMaxStealCounters);
  if (e != hipSuccess) {
    free_witness(cfg);
    return from_hip(e);
  }
  cfg->w_tiles = max_tiles;
  cfg->w_programs = max_programs;
  return PGEMM_OK;
}

pgemm_status pgemm_witness_read(pgemm_config* cfg, pgemm_witness* out, void* hip_stream) {
  if (!cfg || !out) return PGEMM_ERR_INVALID;
  if (cfg->w_visits == nullptr) return PGEMM_ERR_INVALID;
  if (out->tiles < 0 || out->tiles > cfg->w_tiles || out->programs < 0 ||
      out->programs > cfg->w_programs)
    return PGEMM_ERR_INVALID;
  DeviceGuard g(cfg->device);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  hipStream_t st = (hipStream_t)hip_stream;
  if (hipStreamSynchronize(st) != hipSuccess) return PGEMM_ERR_DEVICE;
  struct Copy { void* dst; const void* src; size_t bytes; };
  const size_t t = (size_t)out->tiles, p = (size_t)out->programs;
  Copy cps[] = {
      {out->visits, cfg->w_visits, 4 * t},      {out->owner, cfg->w_owner, 4 * t},
      {out->order, cfg->w_order, 4 * t},        {out->t_start, cfg->w_t_start, 8 * p},
      {out->t_end, cfg->w_t_end, 8 * p},        {out->hw_id, cfg->w_hw_id, 4 * p},
      {out->cycles, cfg->w_cycles, 8 * p},
      {out->n_tiles, cfg->w_n_tiles, 4 * p},
      {out->claims, cfg->w_claims, 4 * p * pgk::kMaxStealCounters},
  };
  for (const Copy& c : cps) {
    if (!c.dst || c.bytes == 0) continue;
    if (hipMemcpy(c.dst, c.src, c.bytes, hipMemcpyDeviceToHost) != hipSuccess)
      return PGEMM_ERR_DEVICE;
  }
  if (out->counters) {  // one counter per 256-byte block on the device, dense in the output
    for (int x = 0; x < cfg->capacity; ++x)
      if (hipMemcpy(out->counters + x, cfg->counters + (size_t)x * pgk::kCounterStride, sizeof(int),
                    hipMemcpyDeviceToHost) != hipSuccess)
        return PGEMM_ERR_DEVICE;
  }
  return PGEMM_OK;
}

pgemm_status pgemm_run(pgemm_config* cfg, const void* A, const void* B, void* C, int64_t M,
                       int64_t N, int64_t K, pgemm_dtype dtype, pgemm_sched sched,
                       const pgemm_args* args, void* hip_stream) {
  if (!cfg) return PGEMM_ERR_INVALID;
  return gemm_call(cfg, A, B, C, M, N, K, dtype, sched, args, hip_stream,
                   CallBuffers{cfg->counters, cfg->capacity, &cfg->counters_dirty, cfg->ws, cfg->ws_bytes, true});
}

pgemm_status pgemm_run_noalloc(pgemm_config* cfg, const void* A, const void* B, void* C, int64_t M,
                               int64_t N, int64_t K, pgemm_dtype dtype, pgemm_sched sched,
                               const pgemm_args* args, void* hip_stream) {
  if (!cfg || !cfg->scratch) return PGEMM_ERR_INVALID;
  if (args && (args->debug_flags & PGEMM_DEBUG_WITNESS)) return PGEMM_ERR_UNSUPPORTED;
  return gemm_call(cfg, A, B, C, M, N, K, dtype, sched, args, hip_stream,
                   CallBuffers{reinterpret_cast<int*>(cfg->scratch), kScratchCounters, &g_scratch_dirty[cfg->device],
                               reinterpret_cast<float*>(cfg->scratch + kScratchCounterBytes),
                               kScratchWsBytes, false});
}

}  // extern "C"

namespace {

pgemm_status gemm_call(pgemm_config* cfg, const void* A, const void* B, void* C, int64_t M, int64_t N,
                       int64_t K, pgemm_dtype dtype, pgemm_sched sched, const pgemm_args* args,
                       void* hip_stream, CallBuffers buf) {
  if (!A || !B || !C) return PGEMM_ERR_INVALID;
  GemmChoice ch;
  pgemm_status st = choose_gemm(M, N, K, dtype, sched, args, A, B, C, ch);
  if (st != PGEMM_OK) return st;
  const bool fp8 = ch.kernel == PGEMM_KERNEL_FP8;
  if (fp8 && (!args || !args->a_scale || !args->b_scale)) return PGEMM_ERR_INVALID;
  const int bm = ch.bm, bn = ch.bn;
  const int dev = cfg->device;
  const size_t esz = fp8 ? 1 : 2;
  const size_t csz = dtype == PGEMM_BF16_OUT_F32 ? 4 : 2;
  if (!device_range(A, span_bytes(M, K, esz), dev) || !device_range(B, span_bytes(K, N, esz), dev) ||
      !device_range(C, span_bytes(M, N, csz), dev))
    return PGEMM_ERR_INVALID;
  if (fp8 && (!device_range(args->a_scale, span_bytes(K / 128, M, 1), dev) ||
              !device_range(args->b_scale, span_bytes(K / 128, N, 1), dev)))
    return PGEMM_ERR_INVALID;
  // C must not overlap A or B
  {
    const char* c0 = (const char*)C;
    const char* c1 = c0 + (size_t)M * N * csz;
    const char* a0 = (const char*)A;
    const char* a1 = a0 + (size_t)M * K * esz;
    const char* b0 = (const char*)B;
    const char* b1 = b0 + (size_t)K * N * esz;
    if ((c0 < a1 && a0 < c1) || (c0 < b1 && b0 < c1)) return PGEMM_ERR_INVALID;
  }

  pgk::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = A;
  p.B = B;
  p.C = C;
  p.sa = fp8 ? args->a_scale : nullptr;
  p.sb = fp8 ? args->b_scale : nullptr;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  const int64_t npm = (M + bm - 1) / bm, npn = (N + bn - 1) / bn;
  if (npm > 0x7fffffffLL || npn > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  DeviceGuard g(dev);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  const pgk::KernelInfo ki = gemm_info(ch);
  st = make_sched(cfg, sched, args, (int)npm, (int)npn, cfg->num_cus * ki.occupancy, true, p.s);
  if (st != PGEMM_OK) return st;
  choose_order(cfg, args, p.s, ch.bm, ch.bn, nullptr, 0);
  if (p.s.X > buf.n_counters) return PGEMM_ERR_INVALID;
  p.s.counters = buf.counters;
  const bool sk = sched == PGEMM_SCHED_STREAM_K;
  const size_t ws_need = sk ? (size_t)p.s.G * 2 * (size_t)ch.bm * ch.bn * sizeof(float) : 0;
  if (sk) {
    // stream-K runs on the direct-to-LDS bf16 kernel and the fp8 kernel,
    // without the witness
    if (ch.kernel != PGEMM_KERNEL_BF16_LDS && ch.kernel != PGEMM_KERNEL_FP8) return PGEMM_ERR_UNSUPPORTED;
    if (args && (args->debug_flags & PGEMM_DEBUG_WITNESS)) return PGEMM_ERR_UNSUPPORTED;
    // the static scratch never grows: a grid whose partial sums do not fit is refused
    if (ws_need > buf.ws_bytes && !buf.growable) return PGEMM_ERR_INVALID;
  }
  if (validate_only(args)) return PGEMM_OK;
  hipStream_t stream = (hipStream_t)hip_stream;
  if (sk) {
    if (ws_need > buf.ws_bytes) {
      st = ensure_workspace(cfg, ws_need, stream);
      if (st != PGEMM_OK) return st;
      buf.ws = cfg->ws;
    }
    p.ws = buf.ws;
  }
  bool witness = false;
  st = make_witness(cfg, args, p.s, p.w, witness, stream);
  if (st != PGEMM_OK) return st;
  st = reset_counters(args, p.s, buf.n_counters, buf.dirty, witness, stream);
  if (st != PGEMM_OK) return st;

  hipError_t e;
  if (fp8)
    e = sk ? pgk::launch_gemm_fp8_sk(p, ch.bm, ch.bn, stream)
           : pgk::launch_gemm_fp8(p, ch.bm, ch.bn, ch.bk, true, witness, stream);
  else if (sk)
    e = pgk::launch_gemm_bf16_lds_sk(p, ch.bm, ch.bn, ch.out_bf16, stream);
  else if (ch.kernel == PGEMM_KERNEL_BF16_LDS)
    e = pgk::launch_gemm_bf16_lds(p, ch.bm, ch.bn, ch.out_bf16, witness, stream);
  else if (ch.kernel == PGEMM_KERNEL_BF16_PINGPONG)
    e = pgk::launch_gemm_bf16_pp(p, ch.out_bf16, witness, stream);
  else
    e = pgk::launch_gemm_bf16(p, ch.bm, ch.bn, ch.bk, ch.out_bf16, ch.vec, witness, stream);
  if (e == hipSuccess && sk) {
    pgk::SkFixParams f;
    f.ws = buf.ws;
    f.C = C;
    f.M = (int)M;
    f.N = (int)N;
    f.T = p.s.T;
    f.nk = (int)((K + ch.bk - 1) / ch.bk);
    f.G = p.s.G;
    f.dp = pgs::sk_dp_tiles(p.s.T, p.s.G);
    f.W = (long long)(f.T - f.dp) * f.nk;
    f.num_pid_m = p.s.num_pid_m;
    f.num_pid_n = p.s.num_pid_n;
    f.gs = p.s.gs;
    e = pgk::launch_sk_fixup(f, ch.bm, ch.bn, ch.out_bf16, stream);
  }
  if (e == hipErrorInvalidValue) return PGEMM_ERR_UNSUPPORTED;
  return e == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

pgemm_status padd_run(pgemm_config* cfg, const float* X, const float* Y, float* C, int64_t rows,
                      int64_t cols, int tile_rows, int tile_cols, pgemm_sched sched,
                      const pgemm_args* args, void* hip_stream) {
  if (!cfg || !X || !Y || !C) return PGEMM_ERR_INVALID;
  if (rows < 1 || cols < 1 || rows > 0x7fffffffLL || cols > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  if (tile_rows < 1 || tile_cols < 1) return PGEMM_ERR_INVALID;
  if (!pgk::padd_tile_supported(tile_rows, tile_cols)) return PGEMM_ERR_UNSUPPORTED;
  const int dev = cfg->device;
  const size_t bytes = span_bytes(rows, cols, 4);
  if (!device_range(X, bytes, dev) || !device_range(Y, bytes, dev) || !device_range(C, bytes, dev))
    return PGEMM_ERR_INVALID;
  {
    const char* c0 = (const char*)C;
    const char* xs[2] = {(const char*)X, (const char*)Y};
    for (const char* x0 : xs)
      if (x0 != c0 && c0 < x0 + bytes && x0 < c0 + bytes) return PGEMM_ERR_INVALID;
  }
  pgk::AddParams p;
  memset(&p, 0, sizeof(p));
  p.X = X;
  p.Y = Y;
  p.C = C;
  p.rows = (int)rows;
  p.cols = (int)cols;
  const int64_t npm = (rows + tile_rows - 1) / tile_rows, npn = (cols + tile_cols - 1) / tile_cols;
  if (npm > 0x7fffffffLL || npn > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  const bool vec = (cols % 4 == 0) && aligned(X, 16) && aligned(Y, 16) && aligned(C, 16);
  DeviceGuard g(dev);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  const pgk::KernelInfo ki = pgk::info_padd(tile_rows, tile_cols, vec);
  pgemm_status st = make_sched(cfg, sched, args, (int)npm, (int)npn, cfg->num_cus * ki.occupancy, false, p.s);
  if (st != PGEMM_OK) return st;
  const int step = pgk::padd_tiles_per_step(tile_rows, tile_cols);
  p.s.chunk = step;
  if (args && args->claim_chunk == PGEMM_CLAIM_PAIRS) return PGEMM_ERR_UNSUPPORTED;
  if (args && args->claim_chunk) {
    if (args->claim_chunk < 1 || args->claim_chunk > step) return PGEMM_ERR_INVALID;
    p.s.chunk = args->claim_chunk;
  }
  if (validate_only(args)) return PGEMM_OK;
  hipStream_t stream = (hipStream_t)hip_stream;
  bool witness = false;
  st = make_witness(cfg, args, p.s, p.w, witness, stream);
  if (st != PGEMM_OK) return st;
  st = reset_counters(args, p.s, cfg->capacity, &cfg->counters_dirty, witness, stream);
  if (st != PGEMM_OK) return st;
  hipError_t e = pgk::launch_padd(p, tile_rows, tile_cols, vec, witness, stream);
  if (e == hipErrorInvalidValue) return PGEMM_ERR_UNSUPPORTED;
  return e == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH;
}

pgemm_status pgemm_plan_gemm(pgemm_config* cfg, const void* A, const void* B, const void* C,
                             int64_t M, int64_t N, int64_t K, pgemm_dtype dtype, pgemm_sched sched,
                             const pgemm_args* args, pgemm_plan* out) {
  if (!cfg || !out) return PGEMM_ERR_INVALID;
  GemmChoice ch;
  pgemm_status st = choose_gemm(M, N, K, dtype, sched, args, A, B, C, ch);
  if (st != PGEMM_OK) return st;
  const int64_t npm = (M + ch.bm - 1) / ch.bm, npn = (N + ch.bn - 1) / ch.bn;
  if (npm > 0x7fffffffLL || npn > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  DeviceGuard g(cfg->device);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  const pgk::KernelInfo ki = gemm_info(ch);
  pgk::SchedParams s;
  st = make_sched(cfg, sched, args, (int)npm, (int)npn, cfg->num_cus * ki.occupancy, true, s);
  if (st != PGEMM_OK) return st;
  choose_order(cfg, args, s, ch.bm, ch.bn, nullptr, 0);
  fill_plan(s, ki, ch.bm, ch.bn, ch.bk, ch.kernel, out);
  return PGEMM_OK;
}

pgemm_status pgemm_plan_add(pgemm_config* cfg, const float* X, const float* Y, const float* C,
                            int64_t rows, int64_t cols, int tile_rows, int tile_cols,
                            pgemm_sched sched, const pgemm_args* args, pgemm_plan* out) {
  if (!cfg || !out) return PGEMM_ERR_INVALID;
  if (rows < 1 || cols < 1 || rows > 0x7fffffffLL || cols > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  if (tile_rows < 1 || tile_cols < 1) return PGEMM_ERR_INVALID;
  if (!pgk::padd_tile_supported(tile_rows, tile_cols)) return PGEMM_ERR_UNSUPPORTED;
  const int64_t npm = (rows + tile_rows - 1) / tile_rows, npn = (cols + tile_cols - 1) / tile_cols;
  if (npm > 0x7fffffffLL || npn > 0x7fffffffLL) return PGEMM_ERR_INVALID;
  const bool vec = (cols % 4 == 0) && (!X || aligned(X, 16)) && (!Y || aligned(Y, 16)) &&
                   (!C || aligned(C, 16));
  DeviceGuard g(cfg->device);
  if (!g.ok) return PGEMM_ERR_DEVICE;
  const pgk::KernelInfo ki = pgk::info_padd(tile_rows, tile_cols, vec);
  pgk::SchedParams s;
  pgemm_status st = make_sched(cfg, sched, args, (int)npm, (int)npn, cfg->num_cus * ki.occupancy, false, s);
  if (st != PGEMM_OK) return st;
  fill_plan(s, ki, tile_rows, tile_cols, 0, PGEMM_KERNEL_ADD, out);
  return PGEMM_OK;
}

}  // extern "C"
