/*
 * pgemm.h -- persistent tiled GEMM and persistent 2-D add with tile
 * schedulers, for AMD Instinct MI355X (gfx950).
 *
 * Every entry point is extern "C", takes plain host or device pointers and
 * sizes, returns a pgemm_status and never throws.  Argument errors are
 * reported before anything is enqueued.  Compute calls are asynchronous on
 * the HIP stream passed in (a hipStream_t given as void*; NULL is the null
 * stream); device faults surface at the caller's next synchronisation.
 *
 * Sources for the operations (page title, section):
 *  - "Work Stealing Scheduler Kernel" (tritonBLAS PR #65): overview (an
 *    opt-in per-XCD work-stealing persistent GEMM with preallocated reusable
 *    buffers), review of the matmul wrapper (config object with the CU count
 *    and an int32 tile-counter array sized by max_xcds, counters reset before
 *    every launch, grid = number of CUs, kernel arguments A, B, C, a_scale,
 *    b_scale, tile_counter, M, N, K), review of the kernel (masked edge
 *    tiles, no index wrapping; counter index bounded by the array size).
 *  - "Implement persistent kernels" (Helion PR #238), example output:
 *    persistent blocked, interleaved and L2-grouped schedules of a 2-D add.
 *  - "[Feature] Introduce tile scheduler" (TileLang PR #2441): persistent
 *    scheduler object with a swizzle / group size, block-scaled fp8 GEMM with
 *    scale shape (1, 1, 128) and K-group-major scale arrays.
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PGEMM_API __attribute__((visibility("default")))
#else
#define PGEMM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PGEMM_OK = 0,
  PGEMM_ERR_INVALID = 1,     /* bad argument or state; nothing was enqueued */
  PGEMM_ERR_UNSUPPORTED = 2, /* device is not gfx950, or no kernel built for the request */
  PGEMM_ERR_DEVICE = 3,      /* a HIP runtime call failed */
  PGEMM_ERR_OOM = 4,         /* a device allocation failed */
  PGEMM_ERR_LAUNCH = 5       /* the kernel launch was rejected */
} pgemm_status;

/* Operand / result formats. */
typedef enum {
  /* A, B bf16; fp32 accumulate; C fp32. */
  PGEMM_BF16_OUT_F32 = 0,
  /* A, B bf16; fp32 accumulate; C bf16 (round to nearest even). */
  PGEMM_BF16_OUT_BF16 = 1,
  /* A, B OCP e4m3 bytes with one e8m0 scale byte per 128 consecutive K
   * elements per row of A (a_scale[K/128][M]) and per column of B
   * (b_scale[K/128][N]); value = e4m3(q) * 2^(scale - 127); fp32
   * accumulate; C bf16.  K must be a multiple of 128 (PGEMM_ERR_INVALID
   * otherwise); N a multiple of 16, A, B, C 16-byte aligned, and one tile's
   * panels within 32-bit byte offsets (tile_m*K, 128*N and tile_m*N*2 all
   * below 2^31) (PGEMM_ERR_UNSUPPORTED otherwise). */
  PGEMM_FP8E4M3_B128_OUT_BF16 = 2
} pgemm_dtype;

/* Tile schedulers.  T = number of output tiles, G = grid (programs), X = XCDs.
 * v is a tile id in [0, T); it is decoded into (pid_m, pid_n).
 *  BLOCKED          program p takes [p*ceil(T/G), min((p+1)*ceil(T/G), T)),
 *                   plain decode (pid_m = v mod num_pid_m fastest).
 *  INTERLEAVED      program p takes p, p+G, p+2G, ...; plain decode.
 *  GROUPED          stride-by-grid over the grouped order: group_size rows of
 *                   tiles per group, the last group shortened.
 *  WORK_STEALING    one int32 counter per XCD; program p claims from counter
 *                   p mod X the tiles of the contiguous range
 *                   [floor(x*T/X), floor((x+1)*T/X)) of the grouped order
 *                   until a claim falls past its end.  Needs G >= X.
 *  BLOCKED_GROUPED  blocked ranges over the grouped order.
 *  STREAM_K         the comparator named by "Work Stealing Scheduler
 *                   Kernel" (tritonBLAS PR #65, benchmark harness), taken as
 *                   a data-parallel + stream-K hybrid: every full wave,
 *                   floor(T/G)*G tiles, is data-parallel (stride-by-grid over
 *                   the grouped order), and the K-slabs of the remaining
 *                   T mod G tiles are cut into G equal contiguous runs, each
 *                   at most one tile long.
 *                   Tiles split between runs are summed (fp32, slab order)
 *                   by a fix-up kernel from per-program partial-sum slots in
 *                   a workspace the config allocates on first use (G x 2
 *                   tiles of fp32).  bf16 on the direct-to-LDS kernel
 *                   (aligned operands, K and N multiples of 8) and block-
 *                   scaled fp8, single problems, no witness; otherwise
 *                   PGEMM_ERR_UNSUPPORTED.  Results are deterministic but
 *                   not bitwise equal to the other schedulers on split
 *                   tiles (different summation order).
 *  WORK_STEALING_XCC  work stealing across XCDs, the pages' per-XCD
 *                   counters carried one step further: same counters and
 *                   ranges, but a program's home counter is the hardware XCC
 *                   it runs on (so its tiles stay in that XCD's L2 whatever
 *                   the dispatch order), and once its home range is
 *                   exhausted it reads the counters it has not passed (one
 *                   round of loads), skips those past their range and claims
 *                   from the next one in cyclic order that is not, stopping
 *                   when none is left.  Every tile is still computed exactly
 *                   once and completion does not depend on placement (any
 *                   G >= 1); a program makes one failing claim on its home
 *                   counter and at most one on each other.  Needs X <= 8
 *                   (PGEMM_ERR_UNSUPPORTED otherwise). */
typedef enum {
  PGEMM_SCHED_BLOCKED = 0,
  PGEMM_SCHED_INTERLEAVED = 1,
  PGEMM_SCHED_GROUPED = 2,
  PGEMM_SCHED_WORK_STEALING = 3,
  PGEMM_SCHED_BLOCKED_GROUPED = 4,
  PGEMM_SCHED_STREAM_K = 5,
  PGEMM_SCHED_WORK_STEALING_XCC = 6
} pgemm_sched;

/* debug_flags (tests and measurement only). */
#define PGEMM_DEBUG_WITNESS 0x1u    /* record per-tile visits / owner / order and per-program
                                       timing into the witness buffers (see pgemm_witness_enable) */
#define PGEMM_DEBUG_SKIP_RESET 0x2u /* do not zero the work-stealing counters before the launch */
#define PGEMM_DEBUG_STRAGGLER 0x4u  /* program straggler_program waits straggler_ns before each tile */
#define PGEMM_DEBUG_REGISTER_STAGED 0x8u /* bf16: use the register-staged kernel (the path taken
                                            for unaligned shapes) even where the direct-to-LDS
                                            kernel applies */
#define PGEMM_DEBUG_STRAGGLER_XCC 0x10u /* every program on hardware XCC straggler_program waits
                                           straggler_ns before each tile (not with
                                           PGEMM_DEBUG_STRAGGLER: PGEMM_ERR_INVALID) */
#define PGEMM_DEBUG_VALIDATE_ONLY 0x20u /* check every argument, buffer ranges included, and
                                           return PGEMM_OK without enqueueing anything */

/* claim_chunk value for paired claims (GEMM, both work-stealing kinds): the
 * counter counts claims; with P = ceil(G / X) programs per counter, a range of
 * n tiles hands out pairs of consecutive tiles over its first
 * L = 2 * min(n / 2, P * (ceil(n / P) / 2)) tiles and single tiles after
 * that, so a program computes neighbouring tiles back to back while, with
 * equal speeds, none gets more tiles than under single claims. */
#define PGEMM_CLAIM_PAIRS (-1)

/* Optional per-call arguments; pass NULL for all defaults. */
typedef struct {
  int tile_m, tile_n, tile_k; /* 0 => default: bf16 256x256x64, fp8 256x256x128 */
  int group_size;             /* grouped order rows per group; 0 => 8 for the GEMM, 1 for the
                                 add (memory order: an add has no operand panels to keep in L2,
                                 and tiles side by side in a row spread over the memory channels) */
  int grid;                   /* programs; 0 => G0 = number of CUs x workgroups of the selected
                                 kernel one CU holds at once; the GEMM's data-parallel
                                 schedulers then take the balanced grid: the fewest
                                 programs, a multiple of the XCD count X, that finish in
                                 as many rounds of tiles as G0 (each XCD's ceil(T/X)
                                 tiles over ceil(T/X) / rounds programs); stream-K and
                                 the add keep G0 (see pgemm_plan_gemm) */
  int claim_chunk;            /* tiles per work-stealing claim (consecutive in the counter's
                                 range); GEMM 1..64 or PGEMM_CLAIM_PAIRS, 0 => 1; add 1..U
                                 (tiles a program handles per step), 0 => U */
  const uint8_t* a_scale;     /* fp8: device, e8m0 [K/128][M] */
  const uint8_t* b_scale;     /* fp8: device, e8m0 [K/128][N] */
  unsigned debug_flags;       /* PGEMM_DEBUG_* */
  int straggler_program;      /* with PGEMM_DEBUG_STRAGGLER */
  int straggler_ns;           /* with PGEMM_DEBUG_STRAGGLER */
  int pipeline;               /* bf16 256x256x64 tiles on the direct-to-LDS terms: PGEMM_PIPELINE_*;
                                 0 => PGEMM_PIPELINE_DEFAULT */
  int program_order;          /* GEMM static walks: PGEMM_ORDER_*; 0 => DEFAULT */
} pgemm_args;

/* pgemm_args.program_order: which workgroup plays which program of a GEMM's
 * static walk (BLOCKED, INTERLEAVED, GROUPED, BLOCKED_GROUPED).  The hardware
 * hands the workgroups of a launch to the XCDs round robin (workgroup i to
 * XCD (i + o) mod X, o depending on earlier launches), so the workgroups of
 * one XCD are those of one residue of i mod X.
 *  XCD_MAJOR  when X > 1 divides G, workgroup i plays program
 *             (i mod X) * (G / X) + i / X: the programs of one XCD have
 *             consecutive ids (whatever o is), so in the grouped order the tiles they take in
 *             one round form a compact block whose operand panels meet in
 *             that XCD's L2, as a work-stealing range does; otherwise as
 *             DISPATCH.
 *  DISPATCH   workgroup i plays program i.
 *  DEFAULT    XCD_MAJOR where it makes the programs' first tiles touch fewer
 *             operand panels per XCD (rows of tiles weighted by tile_m plus
 *             columns weighted by tile_n, summed over the XCDs) than
 *             DISPATCH, else DISPATCH (for the plain decode with many rows of
 *             tiles, consecutive ids form a column and the round robin is the
 *             compact assignment); pgemm_plan.xcd_major reports the choice.
 * The set of tiles each program takes, and so C, is the same under all; the
 * witness records programs by this number (owner, per-program arrays).  The
 * work-stealing kinds and stream-K always number programs by workgroup (a
 * work-stealing program's home counter is the XCD it runs on), and so does
 * the add. */
#define PGEMM_ORDER_DEFAULT 0
#define PGEMM_ORDER_DISPATCH 1
#define PGEMM_ORDER_XCD_MAJOR 2

/* pgemm_args.pipeline: how the bf16 256x256x64 kernel feeds its matrix cores.
 *  FOUR_WAVE  four waves, one per SIMD, each owning a 128x128 sub-tile; loads,
 *             LDS reads and MFMAs interleaved in each wave's own stream.
 *  PINGPONG   eight waves, two per SIMD, in two groups that alternate between
 *             matrix work and memory work every two k-steps (one group's LDS
 *             reads, loads and epilogue run under the other group's MFMAs);
 *             the AMD form of the warp-role pipeline of "[Feature] Introduce
 *             tile scheduler" (TileLang PR #2441, MXFP8 example).  Single
 *             problems under every scheduler but STREAM_K (which, like
 *             pgemm_run_grouped, keeps the four-wave kernel).
 * Both give bit-identical C: the per-tile K order is the same. */
#define PGEMM_PIPELINE_DEFAULT 0
#define PGEMM_PIPELINE_FOUR_WAVE 1
#define PGEMM_PIPELINE_PINGPONG 2

typedef struct pgemm_config pgemm_config; /* opaque */

typedef struct {
  int num_cus;           /* compute units (grid size of a default launch) */
  int num_xcds;          /* XCDs = number of work-stealing counters in use */
  int counter_capacity;  /* length of the int32 counter array */
  int wall_clock_khz;    /* tick rate of the witness timestamps */
  int clock_khz;         /* peak engine clock */
  int lds_bytes_per_cu;  /* LDS per compute unit */
  char arch[64];         /* gcnArchName */
} pgemm_info;

/* Create a configuration for HIP device `device`: reads the CU count and the
 * XCD count, allocates and zeroes an int32 work-stealing counter array of
 * max_xcds entries (0 => 16), and allocates the stream-K workspace for the
 * default grid of every stream-K tile (two fp32 tiles per program:
 * CUs x 512 KiB at 256x256 tiles, 128 MiB on 256 CUs).  Fails with PGEMM_ERR_INVALID if the device has more XCDs than max_xcds
 * (the counter index p mod X would run past the array), with
 * PGEMM_ERR_UNSUPPORTED if the device is not gfx950.  *out receives the new
 * config, owned by the caller until pgemm_config_destroy. */
PGEMM_API pgemm_status pgemm_config_create(int device, int max_xcds, pgemm_config** out);

/* Device facts read at creation. */
PGEMM_API pgemm_status pgemm_config_query(const pgemm_config* cfg, pgemm_info* info);

/* Free the counters and witness buffers (after the caller has synchronised
 * the streams that used them).  NULL is a no-op. */
PGEMM_API pgemm_status pgemm_config_destroy(pgemm_config* cfg);

/* C[M][N] = A[M][K] . B[K][N], all dense row-major on device `cfg`'s GPU.
 * A, B, C: device pointers owned by the caller; C must not alias A or B.
 * Elements of C outside [0, M) x [0, N) are never written.  With either
 * work-stealing scheduler the counters are zeroed on `hip_stream` first.
 * bf16 shapes the direct-to-LDS kernel cannot take (unaligned pointers, K
 * or N not a multiple of 8, a tile's panels past 32-bit byte offsets) run
 * on the register-staged kernel, which addresses with 64-bit offsets.
 * A config holds one counter array: calls with the same config on different
 * streams must not overlap.  A config also keeps host-side state between
 * calls (whether its counters may be dirty, its stream-K workspace, the last
 * program-numbering decision), so one config serves one host thread at a
 * time; threads that call concurrently use a config each.  Errors: NULL pointer, M, N or K < 1,
 * group_size < 1, grid < 1 (or < X for work stealing), fp8 without scales or
 * with K % 128 != 0 => PGEMM_ERR_INVALID; a buffer whose byte range (A:
 * M*K, B: K*N elements, C: M*N, scales: (K/128)*M and (K/128)*N bytes) does
 * not lie inside one device allocation of the config's device =>
 * PGEMM_ERR_INVALID (the kernels address by the sizes given, so a shorter
 * buffer would be accessed past its end); tile shape not built =>
 * PGEMM_ERR_UNSUPPORTED.  PGEMM_SCHED_STREAM_K uses the workspace the config
 * allocated; only a grid larger than the default (args->grid) grows it,
 * after a device synchronisation (PGEMM_ERR_OOM if that fails, and
 * PGEMM_ERR_INVALID while the stream is being captured). */
PGEMM_API pgemm_status pgemm_run(pgemm_config* cfg, const void* A, const void* B, void* C,
                       int64_t M, int64_t N, int64_t K, pgemm_dtype dtype,
                       pgemm_sched sched, const pgemm_args* args, void* hip_stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results (bit for bit), errors and stream rules as pgemm_run,
 * but the work-stealing counters and the stream-K partial sums live in a
 * static device array of PGEMM_NOALLOC_SCRATCH_BYTES on each device (held
 * from the first pgemm_config_create on that device until the process ends)
 * instead of the config's buffers, so the call allocates nothing at any
 * grid.  Limits: stream-K's partial sums, grid x 2 x tile_m x tile_n x 4
 * bytes, must fit in 64 MiB (the default grid fits at 128x128 and 128x256
 * tiles; at 256x256 tiles pass args->grid <= 128), otherwise
 * PGEMM_ERR_INVALID with nothing enqueued; at most 16 XCDs; no witness
 * (PGEMM_ERR_UNSUPPORTED).  Every call on a GPU uses that GPU's one array,
 * which keeps the last call's contents (the counters are cleared on the
 * stream before each work-stealing launch): calls that overlap in time on
 * one GPU, from any stream or config, race and must not be made. */
#define PGEMM_NOALLOC_SCRATCH_BYTES ((64u << 20) + 4096u)
PGEMM_API pgemm_status pgemm_run_noalloc(pgemm_config* cfg, const void* A, const void* B, void* C,
                               int64_t M, int64_t N, int64_t K, pgemm_dtype dtype,
                               pgemm_sched sched, const pgemm_args* args, void* hip_stream);

/* C[rows][cols] = X + Y (fp32, one IEEE add per element, round to nearest
 * even), persistent over tile_rows x tile_cols tiles with the same
 * schedulers (tile rows are dimension 0 of the decode).  Built tiles: 32x16,
 * 64x64, 128x128.  Same ownership, error and stream rules as pgemm_run (X,
 * Y and C must each span rows*cols floats inside one device allocation).
 * C may alias X or Y exactly (in place), not partially. */
PGEMM_API pgemm_status padd_run(pgemm_config* cfg, const float* X, const float* Y, float* C,
                      int64_t rows, int64_t cols, int tile_rows, int tile_cols,
                      pgemm_sched sched, const pgemm_args* args, void* hip_stream);

/* Several GEMMs in one persistent launch, the multi-problem loop of
 * "Implement persistent kernels" (Helion PR #238, multi-loop listings)
 * applied to the GEMM (a grouped GEMM): problem g's output tiles take the
 * virtual tile ids from the sum of the earlier problems' tile counts on, the
 * scheduler walks the shared space, and the persistent programs move from
 * one problem's tile to another's without a new launch.  `problems` is a host
 * array of `count` entries (1..PGEMM_MAX_PROBLEMS), read during the call.
 * bf16 (PGEMM_BF16_OUT_F32 / _OUT_BF16) on the direct-to-LDS kernel's terms
 * (A, B, C 16-byte aligned, K and N multiples of 8), or block-scaled fp8
 * (PGEMM_FP8E4M3_B128_OUT_BF16, each problem with its own a_scale / b_scale,
 * K a multiple of 128, N of 16); otherwise PGEMM_ERR_UNSUPPORTED.  One tile
 * shape for all problems (args->tile_*; args->a_scale / b_scale unused); M
 * or N may be 0, K >= 1.  Every scheduler but
 * STREAM_K (PGEMM_ERR_UNSUPPORTED).  No C may overlap any operand or
 * another C (PGEMM_ERR_INVALID).  Each problem's C is bit-identical to a
 * pgemm_run of that problem with the same tile.  The witness indexes tiles
 * by virtual id. */
#define PGEMM_MAX_PROBLEMS 8
typedef struct {
  const void* A;   /* device, bf16 or e4m3 [M][K] */
  const void* B;   /* device, bf16 or e4m3 [K][N] */
  void* C;         /* device, [M][N] of the dtype's output type */
  int64_t M, N, K;
  const uint8_t* a_scale;  /* fp8: device, e8m0 [K/128][M]; otherwise ignored */
  const uint8_t* b_scale;  /* fp8: device, e8m0 [K/128][N]; otherwise ignored */
} pgemm_problem;

PGEMM_API pgemm_status pgemm_run_grouped(pgemm_config* cfg, const pgemm_problem* problems, int count,
                               pgemm_dtype dtype, pgemm_sched sched, const pgemm_args* args,
                               void* hip_stream);

/* Several adds in one persistent launch ("Implement persistent kernels",
 * Helion PR #238, the multi-loop listings: two problems share one virtual
 * program-id space, ids past the first problem's tile count are reduced by
 * it and decoded in the second).  Here up to PADD_MAX_PROBLEMS problems:
 * problem g owns the virtual tile ids from the sum of the earlier problems'
 * tile counts on; the scheduler walks the shared space (work stealing: the
 * XCD ranges split the shared space) and each id is decoded within its
 * problem as padd_run decodes a single problem.  `problems` is a host array
 * of `count` entries (1..PADD_MAX_PROBLEMS), read during the call.  rows or
 * cols may be 0 (the problem has no tiles).  Each C may alias its own X or
 * Y exactly; any other overlap of a C with a buffer of any problem is
 * PGEMM_ERR_INVALID (the order of problems is not defined).  The witness
 * indexes tiles by virtual id. */
#define PADD_MAX_PROBLEMS 8
typedef struct {
  const float* X;  /* device, [rows][cols] */
  const float* Y;  /* device, [rows][cols] */
  float* C;        /* device, [rows][cols] */
  int64_t rows, cols;
} padd_problem;

PGEMM_API pgemm_status padd_run_multi(pgemm_config* cfg, const padd_problem* problems, int count,
                            int tile_rows, int tile_cols, pgemm_sched sched,
                            const pgemm_args* args, void* hip_stream);

/* Witness buffers for PGEMM_DEBUG_WITNESS launches: per tile (up to
 * max_tiles) visit count, owner program and position in the owner's
 * sequence; per program (up to max_programs) start / end wall-clock ticks,
 * shader clock cycles, hardware id, tile count and, under work stealing, the
 * claims it made on each counter.  Allocated on device by this call and owned by
 * the config. */
PGEMM_API pgemm_status pgemm_witness_enable(pgemm_config* cfg, int64_t max_tiles, int max_programs);

typedef struct {      /* host arrays supplied by the caller */
  int32_t* visits;    /* [tiles] */
  int32_t* owner;     /* [tiles] */
  int32_t* order;     /* [tiles] */
  int64_t tiles;      /* entries to copy */
  int64_t* t_start;   /* [programs] wall-clock ticks */
  int64_t* t_end;     /* [programs] */
  int32_t* hw_id;     /* [programs] bits 0-15: HW_ID register low half; bits 16-19: XCC id */
  int32_t* n_tiles;   /* [programs] */
  int32_t programs;   /* entries to copy */
  int32_t* counters;  /* [counter_capacity] work-stealing counters after the launch */
  int64_t* cycles;    /* [programs] shader clock cycles from program start to end; divided by
                         (t_end - t_start) / wall_clock_khz it is the clock the program ran at */
  int32_t* claims;    /* [programs][8] work-stealing claims (counter increments) each program made
                         on counters 0..7, failing ones included; zero for the static kinds */
} pgemm_witness;

/* Synchronise `hip_stream` and copy the witness of the last launch into the
 * caller's host arrays (any array may be NULL to skip it). */
PGEMM_API pgemm_status pgemm_witness_read(pgemm_config* cfg, pgemm_witness* out, void* hip_stream);

/* Which kernel a call runs. */
typedef enum {
  PGEMM_KERNEL_BF16_LDS = 0,     /* bf16, direct-to-LDS loads (16-byte aligned, K and N % 8 == 0) */
  PGEMM_KERNEL_BF16_STAGED = 1,  /* bf16, register-staged (any shape and alignment) */
  PGEMM_KERNEL_FP8 = 2,          /* block-scaled fp8 */
  PGEMM_KERNEL_ADD = 3,          /* persistent add */
  PGEMM_KERNEL_BF16_PINGPONG = 4 /* bf16, eight waves in ping-pong (PGEMM_PIPELINE_PINGPONG) */
} pgemm_kernel;

/* Launch a call would make.  A persistent launch runs one program per
 * resident workgroup slot: grid = number of CUs x occupancy unless
 * args->grid overrides it (e.g. 128x128 GEMM tiles fit two workgroups per
 * CU, 256x256 tiles one; the add runs one 1024-thread program per CU). */
typedef struct {
  int grid;          /* programs */
  int occupancy;     /* workgroups of the kernel one CU holds at once */
  int64_t tiles;     /* output tiles T */
  int tile_m, tile_n, tile_k;  /* tile_k = 0 for the add */
  int threads;       /* per workgroup */
  int lds_bytes;     /* dynamic LDS per workgroup */
  pgemm_kernel kernel;
  int xcd_major;     /* 1: programs numbered XCD-major (see pgemm_args.program_order) */
} pgemm_plan;

/* The launch pgemm_run would make with the same arguments (no pointer is
 * dereferenced; NULL pointers count as 16-byte aligned).  Same argument
 * errors as pgemm_run, except that fp8 scales are not required. */
PGEMM_API pgemm_status pgemm_plan_gemm(pgemm_config* cfg, const void* A, const void* B, const void* C,
                             int64_t M, int64_t N, int64_t K, pgemm_dtype dtype,
                             pgemm_sched sched, const pgemm_args* args, pgemm_plan* out);

/* The launch padd_run would make with the same arguments (NULL pointers
 * count as 16-byte aligned). */
PGEMM_API pgemm_status pgemm_plan_add(pgemm_config* cfg, const float* X, const float* Y, const float* C,
                            int64_t rows, int64_t cols, int tile_rows, int tile_cols,
                            pgemm_sched sched, const pgemm_args* args, pgemm_plan* out);

/* Static string for a status code. */
PGEMM_API const char* pgemm_status_str(pgemm_status s);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
