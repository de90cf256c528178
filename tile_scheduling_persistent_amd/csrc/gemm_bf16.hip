// Persistent bf16 GEMM for gfx950: C[M][N] = A[M][K] . B[K][N], fp32
// accumulate, fp32 or bf16 C.
//
// One workgroup of 256 threads (4 waves, 2 x 2) per compute unit loops over
// output tiles chosen by the tile scheduler ("Work Stealing Scheduler
// Kernel", tritonBLAS PR #65: grid = number of CUs, per-XCD counters;
// "Implement persistent kernels", Helion PR #238: blocked / interleaved /
// grouped walks).  Per tile:
//  * K is walked in BK = 64 slabs.  Slab k+1 is fetched from global memory
//    into registers with 16-byte buffer loads while the MFMAs consume slab k
//    from LDS; the registers are then written to the other LDS buffer
//    (double buffering, one barrier per slab).  The first slab of the next
//    tile is fetched during the last slab of the current one, so the
//    epilogue overlaps the next tile's loads (the pipeline phase runs on
//    across tiles, as the scheduler's iteration counter does in "[Feature]
//    Introduce tile scheduler", TileLang PR #2441).
//  * Loads go through buffer resources rebased on every slab, so that all
//    per-thread offsets are 32-bit loop invariants and rows past M or K read
//    as zero through the hardware range check; columns past N and the K tail
//    are masked by pointing the offset out of range.  Edge tiles are never
//    wrapped (review of the work-stealing kernel in tritonBLAS PR #65).
//  * A is stored in LDS as [m][k], B transposed as [n][k] (k contiguous, as
//    the MFMA operands want); the transpose of B happens in registers on the
//    way in (8 x 8 blocks of bf16).  16-byte chunks of each LDS row are
//    XOR-swizzled by the row index so that both the row-wise writes and the
//    column-wise operand reads spread over all banks.
//  * Each wave owns a (BM/2) x (BN/2) sub-tile as 32 x 32 MFMA blocks
//    (v_mfma_f32_32x32x16_bf16) with the B^T block as the first operand, so
//    a lane's 4 consecutive accumulators are 4 consecutive columns of C and
//    the epilogue stores 16 bytes (fp32) or 8 bytes (bf16) per lane.
#include "common.hpp"

namespace pgk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr unsigned kOob = 0x80000000u;          // offset past every range
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format

template <int BM, int BN, int BK>
struct Shape {
  static_assert(BK == 64, "bf16 slabs are 64 deep (8 swizzled 16-byte chunks per row)");
  static constexpr int WM = 2, WN = 2;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  static constexpr int SM = TM / 32, SN = TN / 32;  // 32x32 blocks per wave
  static constexpr int CK = BK / 8;                 // 16-byte chunks per LDS row
  static constexpr int A_CHUNKS = BM * CK / kThreads;
  static constexpr int B_BLOCKS = CK * (BN / 8);    // 8x8 blocks per B slab
  static constexpr int B_PER_THREAD = (B_BLOCKS + kThreads - 1) / kThreads;
  static constexpr int A_STAGE = BM * BK;           // elements per LDS stage
  static constexpr int B_STAGE = BN * BK;
  static constexpr int STAGE_BYTES = (A_STAGE + B_STAGE) * 2;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES + 16;
  static_assert(A_CHUNKS * kThreads == BM * CK, "A slab must split evenly");
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// Buffer resource over [base, base + bytes).  base and bytes are uniform
// across the wave; readfirstlane states that, so the resource lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  void* ub = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 8 bf16 starting at p with `count` valid elements (scalar path).
__device__ __forceinline__ u32x4 load8_scalar(const unsigned short* p, int count) {
  unsigned e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = i < count ? (unsigned)p[i] : 0u;
  return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
               e[6] | (e[7] << 16)};
}

__device__ __forceinline__ unsigned lo_pair(unsigned a, unsigned b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ unsigned hi_pair(unsigned a, unsigned b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// v[i] = 8 columns of row i; returns w[j] = 8 rows of column j.
__device__ __forceinline__ void transpose8x8(const u32x4 (&v)[8], u32x4 (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = j >> 1;
    unsigned o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (j & 1) ? hi_pair(v[2 * q][d], v[2 * q + 1][d]) : lo_pair(v[2 * q][d], v[2 * q + 1][d]);
    w[j] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <int BM, int BN, int BK, bool OUT_BF16, bool VEC, bool WITNESS>
__global__ void __launch_bounds__(kThreads) gemm_bf16_kernel(GemmParams P) {
  using S = Shape<BM, BN, BK>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* s_tile = reinterpret_cast<int*>(smem + 2 * S::STAGE_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::WN;
  const int wn = wave % S::WN;
  const int prog = pgs::program_of(blockIdx.x, P.s.G, P.s.X, P.s.xcd_major);
  const int M = P.M, N = P.N, K = P.K;
  const unsigned short* __restrict__ A = static_cast<const unsigned short*>(P.A);
  const unsigned short* __restrict__ B = static_cast<const unsigned short*>(P.B);

  Walker walker(P.s, prog);
  if (WITNESS) walker.claim_row = P.w.claims + (size_t)prog * kMaxStealCounters;
  long long t_start = 0, c_start = 0;
  if (WITNESS && tid == 0) {
    t_start = wall_ticks();
    c_start = shader_cycles();
  }

  // ---- per-thread loop invariants -------------------------------------
  // A staging: chunk q = r*256 + tid -> row q/CK, 16-byte chunk q%CK.
  const int a_c = tid % S::CK;
  const int a_row0 = tid / S::CK;                       // + r * (256 / CK)
  // B staging: 8x8 block blk = b*256 + tid -> k chunk blk%CK, n block blk/CK.
  const int b_kc = tid % S::CK;
  const int b_nb0 = tid / S::CK;                        // + b * (256 / CK)
  // LDS byte offset of the first staging write; chunk r adds r*(256/CK) rows,
  // which leaves the swizzle (row mod 8) unchanged.
  const unsigned a_wr0 = (unsigned)(a_row0 * BK + swz(a_row0, a_c) * 8) * 2u;
  constexpr unsigned kAWrStep = (kThreads / S::CK) * BK * 2;
  // LDS byte offsets of the MFMA operand reads (sub-tile s adds s*32 rows)
  const int r32 = lane & 31;
  unsigned rd_a[BK / 16], rd_b[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int c = kk * 2 + (lane >> 5);
    const int ra = wm * S::TM + r32, rb = wn * S::TN + r32;
    rd_a[kk] = (unsigned)(ra * BK + swz(ra, c) * 8) * 2u;
    rd_b[kk] = (unsigned)(S::A_STAGE * 2) + (unsigned)(rb * BK + swz(rb, c) * 8) * 2u;
  }
  // global byte offsets relative to the per-slab buffer bases
  const unsigned a_gl0 = (unsigned)a_row0 * (unsigned)K * 2u + (unsigned)a_c * 16u;
  const unsigned a_gl_step = (unsigned)(kThreads / S::CK) * (unsigned)K * 2u;
  const unsigned b_gl0 = (unsigned)(b_kc * 8) * (unsigned)N * 2u;
  const unsigned b_gl_step = (unsigned)N * 2u;

  u32x4 ra[S::A_CHUNKS];
  u32x4 rb[S::B_PER_THREAD][8];

  // Fetch the slab (m0, n0, k0) into registers.
  auto gload = [&](int m0, int n0, int k0) {
    if (VEC) {
      const int rows = (M - m0) < BM ? (M - m0) : BM;
      const auto rA = rsrc(A + (size_t)m0 * K + k0, (unsigned)(rows * K - k0) * 2u);
      const bool a_tail = k0 + a_c * 8 >= K;
#pragma unroll
      for (int r = 0; r < S::A_CHUNKS; ++r) ra[r] = bload16(rA, a_tail ? kOob : a_gl0 + r * a_gl_step);
      const int krows = (K - k0) < BK ? (K - k0) : BK;
      const auto rB = rsrc(B + (size_t)k0 * N + n0, (unsigned)(krows * N - n0) * 2u);
#pragma unroll
      for (int b = 0; b < S::B_PER_THREAD; ++b) {
        const int nb = b_nb0 + b * (kThreads / S::CK);
        const bool live = (b * kThreads + tid < S::B_BLOCKS) && (n0 + nb * 8 < N);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[b][i] = bload16(rB, live ? b_gl0 + i * b_gl_step + nb * 16u : kOob);
      }
    } else {
#pragma unroll
      for (int r = 0; r < S::A_CHUNKS; ++r) {
        const int gm = m0 + a_row0 + r * (kThreads / S::CK), gk = k0 + a_c * 8;
        const int cnt = (gm < M) ? K - gk : 0;
        ra[r] = load8_scalar(A + (size_t)(gm < M ? gm : 0) * K + (gk < K ? gk : 0), cnt > 8 ? 8 : cnt);
      }
#pragma unroll
      for (int b = 0; b < S::B_PER_THREAD; ++b) {
        const int nb = b_nb0 + b * (kThreads / S::CK);
        const int gn = n0 + nb * 8;
        const bool live = b * kThreads + tid < S::B_BLOCKS;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int gk = k0 + b_kc * 8 + i;
          const int cnt = (live && gk < K) ? N - gn : 0;
          rb[b][i] = load8_scalar(B + (size_t)(gk < K ? gk : 0) * N + (gn < N ? gn : 0), cnt > 8 ? 8 : cnt);
        }
      }
    }
  };

  // Write the staged registers into LDS stage `st`.
  auto swrite = [&](int st) {
    unsigned char* base = smem + st * S::STAGE_BYTES;
#pragma unroll
    for (int r = 0; r < S::A_CHUNKS; ++r) *reinterpret_cast<u32x4*>(base + a_wr0 + r * kAWrStep) = ra[r];
    unsigned char* bbase = base + S::A_STAGE * 2;
#pragma unroll
    for (int b = 0; b < S::B_PER_THREAD; ++b) {
      if (b * kThreads + tid < S::B_BLOCKS) {
        const int nb = b_nb0 + b * (kThreads / S::CK);
        u32x4 w[8];
        transpose8x8(rb[b], w);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = nb * 8 + j;
          *reinterpret_cast<u32x4*>(bbase + (row * BK + swz(row, b_kc) * 8) * 2) = w[j];
        }
      }
    }
  };

  f32x16 acc[S::SN][S::SM];

  auto compute = [&](int st) {
    const unsigned char* base = smem + st * S::STAGE_BYTES;
    bf16x8 bf[2][S::SN], af[2][S::SM];
    auto frag = [&](int kk, int slot) {
#pragma unroll
      for (int s = 0; s < S::SN; ++s)
        bf[slot][s] = *reinterpret_cast<const bf16x8*>(base + rd_b[kk] + s * 32 * BK * 2);
#pragma unroll
      for (int s = 0; s < S::SM; ++s)
        af[slot][s] = *reinterpret_cast<const bf16x8*>(base + rd_a[kk] + s * 32 * BK * 2);
    };
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) frag(kk + 1, cur ^ 1);
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn)
#pragma unroll
        for (int sm = 0; sm < S::SM; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cur][sn], af[cur][sm],
                                                                acc[sn][sm], 0, 0, 0);
    }
  };

  auto epilogue = [&](int m0, int n0) {
    constexpr unsigned esz = OUT_BF16 ? 2u : 4u;
    if (VEC) {
      const int rows = (M - m0) < BM ? (M - m0) : BM;
      const auto rC = rsrc(static_cast<unsigned char*>(P.C) + ((size_t)m0 * N + n0) * esz,
                           (unsigned)((size_t)rows * N - n0) * esz);
      // lane (r0, c0) of the wave's first block; block (sm, sn), group g adds
      // sm*32 rows and sn*32 + 8g columns.  Rows past M fall outside rC.
      const int r0 = wm * S::TM + (lane & 31);
      const int c0 = wn * S::TN + 4 * (lane >> 5);
      const unsigned eb = (unsigned)(r0 * N + c0) * esz;
      const unsigned rstep = 32u * (unsigned)N * esz;
      const int ncols = N - n0;  // columns of this tile inside C
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm) {
#pragma unroll
        for (int sn = 0; sn < S::SN; ++sn) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int cc = sn * 32 + 8 * g;
            const unsigned off = (c0 + cc < ncols) ? eb + sm * rstep + (unsigned)cc * esz : kOob;
            const f32x16& a = acc[sn][sm];
            if (OUT_BF16) {
              const u32x2 v = u32x2{pack_bf16x2(a[4 * g], a[4 * g + 1]),
                                    pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
              __builtin_amdgcn_raw_buffer_store_b64(v, rC, off, 0, 0);
            } else {
              const f32x4 v = f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rC, off, 0, 0);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm) {
        const int m = m0 + wm * S::TM + sm * 32 + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int sn = 0; sn < S::SN; ++sn) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * S::TN + sn * 32 + 8 * g + 4 * (lane >> 5);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (n + e >= N) continue;
              const float v = acc[sn][sm][4 * g + e];
              if (OUT_BF16)
                static_cast<unsigned short*>(P.C)[(size_t)m * N + n + e] =
                    (unsigned short)(pack_bf16x2(v, 0.0f) & 0xffffu);
              else
                static_cast<float*>(P.C)[(size_t)m * N + n + e] = v;
            }
          }
        }
      }
    }
  };

  const int nk = (K + BK - 1) / BK;
  if (tid == 0) s_tile[0] = walker.first();
  __syncthreads();
  int tile = __builtin_amdgcn_readfirstlane(s_tile[0]);
  int stage = 0;
  int it = 0;
  if (tile >= 0) {
    int pm, pn;
    walker.tile_coords(tile, pm, pn);
    gload(pm * BM, pn * BN, 0);
    swrite(0);
  }
  __syncthreads();

  while (tile >= 0) {
    int pm, pn;
    walker.tile_coords(tile, pm, pn);
    const int m0 = pm * BM, n0 = pn * BN;
    if (tid == 0) {
      if (WITNESS) {
        atomicAdd(P.w.visits + tile, 1);
        P.w.owner[tile] = prog;
        P.w.order[tile] = it;
      }
      if (is_straggler(P.s, prog)) spin_ns(P.s.straggler_ns, P.s.wall_khz);
    }
#pragma unroll
    for (int sn = 0; sn < S::SN; ++sn)
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[sn][sm][e] = 0.0f;

    const int slot = (it + 1) & 1;
    // the claim of the next tile is issued one slab before the last
    if (nk == 1 && tid == 0) s_tile[slot] = walker.next(tile);
    // steady state: slabs 0 .. nk-2, each fetching slab kb+1 of this tile
    for (int kb = 0; kb + 1 < nk; ++kb) {
      if (kb == nk - 2 && tid == 0) s_tile[slot] = walker.next(tile);
      gload(m0, n0, (kb + 1) * BK);
      compute(stage);
      swrite(stage ^ 1);
      __syncthreads();
      stage ^= 1;
    }
    // last slab: fetch the first slab of the next tile (if known already)
    int next = -1;
    if (nk >= 2) {
      next = __builtin_amdgcn_readfirstlane(s_tile[slot]);
      if (next >= 0) {
        int qm, qn;
        walker.tile_coords(next, qm, qn);
        gload(qm * BM, qn * BN, 0);
      }
    }
    compute(stage);
    if (nk >= 2 && next >= 0) swrite(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    epilogue(m0, n0);
    if (nk == 1) {
      next = __builtin_amdgcn_readfirstlane(s_tile[slot]);
      if (next >= 0) {
        int qm, qn;
        walker.tile_coords(next, qm, qn);
        gload(qm * BM, qn * BN, 0);
        swrite(stage);
      }
      __syncthreads();
    }
    tile = next;
    ++it;
  }

  if (WITNESS && tid == 0) {
    P.w.t_start[prog] = t_start;
    P.w.t_end[prog] = wall_ticks();
    P.w.cycles[prog] = shader_cycles() - c_start;
    P.w.hw_id[prog] = hw_placement();
    P.w.n_tiles[prog] = it;
  }
}

template <int BM, int BN, int BK, bool OUT_BF16, bool VEC, bool WITNESS>
hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  using S = Shape<BM, BN, BK>;
  auto kern = gemm_bf16_kernel<BM, BN, BK, OUT_BF16, VEC, WITNESS>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.s.G), dim3(kThreads), S::LDS_BYTES, stream, p);
  return hipGetLastError();
}

template <int BM, int BN, int BK>
hipError_t launch_tile(const GemmParams& p, bool out_bf16, bool vec, bool witness,
                       hipStream_t stream) {
  if (out_bf16) {
    if (vec) return witness ? launch_one<BM, BN, BK, true, true, true>(p, stream)
                            : launch_one<BM, BN, BK, true, true, false>(p, stream);
    return witness ? launch_one<BM, BN, BK, true, false, true>(p, stream)
                   : launch_one<BM, BN, BK, true, false, false>(p, stream);
  }
  if (vec) return witness ? launch_one<BM, BN, BK, false, true, true>(p, stream)
                          : launch_one<BM, BN, BK, false, true, false>(p, stream);
  return witness ? launch_one<BM, BN, BK, false, false, true>(p, stream)
                 : launch_one<BM, BN, BK, false, false, false>(p, stream);
}

template <int BM, int BN, int BK, bool OUT_BF16, bool VEC>
KernelInfo info_one() {
  using S = Shape<BM, BN, BK>;
  static const KernelInfo ki = {
      kThreads, S::LDS_BYTES,
      occupancy_of(reinterpret_cast<const void*>(gemm_bf16_kernel<BM, BN, BK, OUT_BF16, VEC, false>),
                   kThreads, S::LDS_BYTES)};
  return ki;
}

template <int BM, int BN, int BK>
KernelInfo info_tile(bool out_bf16, bool vec) {
  if (out_bf16) return vec ? info_one<BM, BN, BK, true, true>() : info_one<BM, BN, BK, true, false>();
  return vec ? info_one<BM, BN, BK, false, true>() : info_one<BM, BN, BK, false, false>();
}

}  // namespace

KernelInfo info_gemm_bf16(int bm, int bn, int bk, bool out_bf16, bool vec) {
  if (bm == 256 && bn == 256 && bk == 64) return info_tile<256, 256, 64>(out_bf16, vec);
  if (bm == 128 && bn == 128 && bk == 64) return info_tile<128, 128, 64>(out_bf16, vec);
  return KernelInfo{0, 0, 0};
}

bool gemm_bf16_tile_supported(int bm, int bn, int bk) {
  return bk == 64 && ((bm == 256 && bn == 256) || (bm == 128 && bn == 128));
}

// Largest K and N for which the 32-bit buffer offsets of a tile stay in range.
bool gemm_bf16_vec_fits(int bm, int bk, long long N, long long K) {
  return (long long)bm * K * 2 < (1LL << 31) && (long long)bk * N * 2 < (1LL << 31) &&
         (long long)bm * N * 4 < (1LL << 31);
}

hipError_t launch_gemm_bf16(const GemmParams& p, int bm, int bn, int bk, bool out_bf16,
                            bool vec, bool witness, hipStream_t stream) {
  if (bm == 256 && bn == 256 && bk == 64)
    return launch_tile<256, 256, 64>(p, out_bf16, vec, witness, stream);
  if (bm == 128 && bn == 128 && bk == 64)
    return launch_tile<128, 128, 64>(p, out_bf16, vec, witness, stream);
  return hipErrorInvalidValue;
}

}  // namespace pgk
