// Persistent element-wise 2-D add for gfx950: C = X + Y in fp32.
//
// "Implement persistent kernels" (Helion PR #238), example output: a grid of
// one program per compute unit walks tiles of TR rows x TC columns (blocked,
// interleaved, or L2-grouped order), decodes each tile id with rows of tiles
// fastest, and does a masked load of x and y, one add, a masked store.  The
// per-XCD work-stealing walk of "Work Stealing Scheduler Kernel" (tritonBLAS
// PR #65) applies unchanged.
//
// The add is bound by HBM bandwidth, so a workgroup of 1024 threads keeps U
// tiles of its sequence in flight at once: every thread issues all its
// 16-byte loads of X and Y for the U tiles before any add, which gives each
// compute unit about 128 KiB of outstanding reads.  Stores stream past the
// caches (nontemporal).  The tiles of a step are the next U tiles the
// scheduler gives the program (for work stealing: one claim of U tiles, and
// the claim for the following step is made once the current step's loads
// are issued, so its latency overlaps theirs).
//
// Several problems in one launch (the multi-loop listings of the same
// page): the problems' tiles share one virtual id space, problem g's ids
// starting at the sum of the earlier problems' tile counts; the scheduler
// walks the shared space, and each id is located in its problem (an
// unrolled comparison against the start ids) and decoded there.
#include "common.hpp"

namespace pgk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 waves per compute unit: enough loads in flight to cover HBM latency
// with one program per CU.
constexpr int kThreads = 1024;

template <int TR, int TC>
struct AddShape {
  static constexpr int F4 = TR * TC / 4;  // float4 per tile
  // tiles per step: ~4 float4 per thread per operand
  static constexpr int U = (4 * kThreads) / F4 > 0 ? (4 * kThreads) / F4 : 1;
  static constexpr int SLOTS = (U * F4 + kThreads - 1) / kThreads;
  // Streaming (nontemporal) loads pay off when a tile row covers whole
  // 128-byte lines; 16-column tiles share lines between neighbouring tiles,
  // which a later step of the same program may still find in cache.
  static constexpr bool NT_LOAD = TC * 4 >= 128;
  static_assert(TC % 4 == 0, "tile columns must be a multiple of 4");
};

// WS: the scheduler is a work-stealing kind (a separate instance, so the
// static walks carry no claim code between their loads and adds).
template <int TR, int TC, bool VEC, bool WITNESS, bool MULTI, bool WS>
__global__ void __launch_bounds__(kThreads) padd_kernel(AddParams P) {
  using S = AddShape<TR, TC>;
  __shared__ int s_claim[2];
  const int tid = threadIdx.x;
  const int prog = blockIdx.x;
  const int rows = P.rows, cols = P.cols;
  constexpr bool ws = WS;
  Walker walker(P.s, prog);
  if (WITNESS) walker.claim_row = P.w.claims + (size_t)prog * kMaxStealCounters;
  long long t_start = 0, c_start = 0;
  if (WITNESS && tid == 0) {
    t_start = wall_ticks();
    c_start = shader_cycles();
  }

  // Static kinds: every thread walks the same sequence itself.  Work
  // stealing: thread 0 claims, the result is shared through LDS.
  int v0;
  if (ws) {
    if (tid == 0) s_claim[0] = walker.claim();
    __syncthreads();
    v0 = s_claim[0];
  } else {
    v0 = walker.first_static();
  }
  int done = 0;  // tiles computed so far by this program
  int step = 0;
  while (v0 >= 0) {
    // tile ids of this step
    int vt[S::U];
    int next_v0 = -1;
    if (ws) {
      const int e = walker.claim_end(v0);
#pragma unroll
      for (int u = 0; u < S::U; ++u) vt[u] = (v0 + u < e) ? v0 + u : -1;
    } else {
      int v = v0;
#pragma unroll
      for (int u = 0; u < S::U; ++u) {
        vt[u] = v;
        if (v >= 0) v = walker.next_static(v);
      }
      next_v0 = v;
    }
    if (WITNESS && tid == 0) {
#pragma unroll
      for (int u = 0; u < S::U; ++u)
        if (vt[u] >= 0) {
          atomicAdd(P.w.visits + vt[u], 1);
          P.w.owner[vt[u]] = prog;
          P.w.order[vt[u]] = done + u;
        }
    }
    if (tid == 0 && is_straggler(P.s, prog)) spin_ns(P.s.straggler_ns, P.s.wall_khz);

    f32x4 xa[S::SLOTS], ya[S::SLOTS];
    long long off[S::SLOTS];
    int cnt[S::SLOTS];
    const float* xb[S::SLOTS];  // several problems: the slot's problem's operands
    const float* yb[S::SLOTS];
    float* cb[S::SLOTS];
#pragma unroll
    for (int j = 0; j < S::SLOTS; ++j) {
      const int idx = j * kThreads + tid;
      const int u = idx / S::F4;
      const int e = idx % S::F4;
      cnt[j] = 0;
      off[j] = 0;
      xb[j] = P.X;
      yb[j] = P.Y;
      cb[j] = P.C;
      if (u < S::U && vt[u] >= 0) {
        int pm, pn, rows_u = rows, cols_u = cols;
        if (MULTI) {
          AddProblem pr = P.prob[0];
#pragma unroll
          for (int q = 1; q < kMaxAddProblems; ++q)
            if (q < P.nprob && vt[u] >= P.prob[q].tile0) pr = P.prob[q];
          pgs::decode(P.s.kind, vt[u] - pr.tile0, pr.npm, pr.npn, P.s.gs, pm, pn);
          rows_u = pr.rows;
          cols_u = pr.cols;
          xb[j] = pr.X;
          yb[j] = pr.Y;
          cb[j] = pr.C;
        } else {
          walker.tile_coords(vt[u], pm, pn);
        }
        const int r = pm * TR + e / (TC / 4);
        const int c = pn * TC + (e % (TC / 4)) * 4;
        if (r < rows_u && c < cols_u) {
          off[j] = (long long)r * cols_u + c;
          cnt[j] = cols_u - c < 4 ? cols_u - c : 4;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < S::SLOTS; ++j) {
      if (VEC) {
        if (cnt[j] > 0) {
          const f32x4* px = reinterpret_cast<const f32x4*>((MULTI ? xb[j] : P.X) + off[j]);
          const f32x4* py = reinterpret_cast<const f32x4*>((MULTI ? yb[j] : P.Y) + off[j]);
          if (S::NT_LOAD) {
            xa[j] = __builtin_nontemporal_load(px);
            ya[j] = __builtin_nontemporal_load(py);
          } else {
            xa[j] = *px;
            ya[j] = *py;
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xa[j][q] = q < cnt[j] ? (MULTI ? xb[j] : P.X)[off[j] + q] : 0.0f;
          ya[j][q] = q < cnt[j] ? (MULTI ? yb[j] : P.Y)[off[j] + q] : 0.0f;
        }
      }
    }
    // Work stealing: the claim for the next step, made after this step's
    // loads are issued.  The returning atomic and the loads share one wait
    // counter, so thread 0's wait for the claim is the wait the adds need
    // anyway and its latency overlaps theirs; before the stores, whose
    // completion the same counter would also wait for.
    if (ws && tid == 0) s_claim[(step + 1) & 1] = walker.claim();
#pragma unroll
    for (int j = 0; j < S::SLOTS; ++j) {
      if (cnt[j] <= 0) continue;
      const f32x4 z = xa[j] + ya[j];
      float* C = MULTI ? cb[j] : P.C;
      if (VEC) {
        __builtin_nontemporal_store(z, reinterpret_cast<f32x4*>(C + off[j]));
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < cnt[j]) C[off[j] + q] = z[q];
      }
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) done += vt[u] >= 0 ? 1 : 0;

    if (ws) {
      __syncthreads();
      v0 = s_claim[(step + 1) & 1];
    } else {
      v0 = next_v0;
    }
    ++step;
  }

  if (WITNESS && tid == 0) {
    P.w.t_start[prog] = t_start;
    P.w.t_end[prog] = wall_ticks();
    P.w.cycles[prog] = shader_cycles() - c_start;
    P.w.hw_id[prog] = hw_placement();
    P.w.n_tiles[prog] = done;
  }
}

template <int TR, int TC, bool MULTI, bool VEC, bool WITNESS>
void launch_kind(const AddParams& p, hipStream_t stream) {
  if (pgs::work_stealing(p.s.kind))
    hipLaunchKernelGGL((padd_kernel<TR, TC, VEC, WITNESS, MULTI, true>), dim3(p.s.G), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((padd_kernel<TR, TC, VEC, WITNESS, MULTI, false>), dim3(p.s.G), dim3(kThreads), 0, stream, p);
}

template <int TR, int TC, bool MULTI>
hipError_t launch_tile(const AddParams& p, bool vec, bool witness, hipStream_t stream) {
  if (vec) {
    if (witness)
      launch_kind<TR, TC, MULTI, true, true>(p, stream);
    else
      launch_kind<TR, TC, MULTI, true, false>(p, stream);
  } else {
    if (witness)
      launch_kind<TR, TC, MULTI, false, true>(p, stream);
    else
      launch_kind<TR, TC, MULTI, false, false>(p, stream);
  }
  return hipGetLastError();
}

__global__ void zero_i32_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

__global__ void fill_i32_kernel(int* p, int n, int value) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = value;
}

// One program per CU: a 1024-thread program already keeps U tiles per step
// in flight, and a second resident program per CU measured 0-40% slower on
// 8192x8192 (more programs contending for the same HBM queues).
template <int TR, int TC, bool VEC>
KernelInfo info_one() {
  static const KernelInfo ki = {kThreads, 0, 1};
  return ki;
}

template <int TR, int TC>
KernelInfo info_tile(bool vec) { return vec ? info_one<TR, TC, true>() : info_one<TR, TC, false>(); }

}  // namespace

int padd_tiles_per_step(int tr, int tc) {
  if (tr == 32 && tc == 16) return AddShape<32, 16>::U;
  if (tr == 64 && tc == 64) return AddShape<64, 64>::U;
  if (tr == 128 && tc == 128) return AddShape<128, 128>::U;
  return 1;
}

bool padd_tile_supported(int tr, int tc) {
  return (tr == 32 && tc == 16) || (tr == 64 && tc == 64) || (tr == 128 && tc == 128);
}

KernelInfo info_padd(int tr, int tc, bool vec) {
  if (tr == 32 && tc == 16) return info_tile<32, 16>(vec);
  if (tr == 64 && tc == 64) return info_tile<64, 64>(vec);
  if (tr == 128 && tc == 128) return info_tile<128, 128>(vec);
  return KernelInfo{0, 0, 0};
}

hipError_t launch_padd(const AddParams& p, int tr, int tc, bool vec, bool witness,
                       hipStream_t stream) {
  if (tr == 32 && tc == 16) return launch_tile<32, 16, false>(p, vec, witness, stream);
  if (tr == 64 && tc == 64) return launch_tile<64, 64, false>(p, vec, witness, stream);
  if (tr == 128 && tc == 128) return launch_tile<128, 128, false>(p, vec, witness, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_padd_multi(const AddParams& p, int tr, int tc, bool vec, bool witness,
                             hipStream_t stream) {
  if (p.nprob < 1 || p.nprob > kMaxAddProblems) return hipErrorInvalidValue;
  if (tr == 32 && tc == 16) return launch_tile<32, 16, true>(p, vec, witness, stream);
  if (tr == 64 && tc == 64) return launch_tile<64, 64, true>(p, vec, witness, stream);
  if (tr == 128 && tc == 128) return launch_tile<128, 128, true>(p, vec, witness, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fill_i32(int* ptr, int n, int value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, stream, ptr, n, value);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int* ptr, int n, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, stream, ptr, n);
  return hipGetLastError();
}

}  // namespace pgk
