// Persistent block-scaled fp8 GEMM for gfx950: C[M][N] (bf16) = A . B with
// A[M][K], B[K][N] OCP e4m3 bytes, one e8m0 scale byte per 128 consecutive K
// elements per row of A (SA[K/128][M]) and per column of B (SB[K/128][N]),
// fp32 accumulate.
//
// The block-scale shape (1, 1, 128) and the K-group-major scale arrays are
// those of the MXFP8 example in "[Feature] Introduce tile scheduler"
// (TileLang PR #2441), where the scales are applied inside the MMA; the
// persistent tile loop and schedulers are those of "Work Stealing Scheduler
// Kernel" (tritonBLAS PR #65) and "Implement persistent kernels" (Helion PR
// #238).  On gfx950 the scales enter v_mfma_scale_f32_32x32x64_f8f6f4: each
// lane passes one e8m0 byte (selected by opsel) for the 32-element K block
// of its row.  A slab is BK = 128 deep, exactly one scale group, so every
// lane passes its row's scale for the slab's group and the assignment of K
// positions to MFMA blocks does not matter.
//
// Data movement as in gemm_bf16_lds.hip: hand-issued buffer_load ... lds
// (lds_dma.hpp; the next slab's loads stay in flight while the current
// slab is read) for A ([m][k],
// 128-byte rows) and B ([k][n]), both chunk-swizzled against LDS bank
// conflicts (swz_a, swz_b); A operands by ds_read_b128, B^T operands by
// ds_read_b64_tr_b8 (within a 16-lane group, lane i points at row
// K0 + i/2, columns N0 + 8*(i%2) .. +7, and lane j receives rows K0 .. K0+7
// of column N0 + j).  Lane l of the MFMA owns logical K positions
// 32*(l/32) .. +31 of each 64-deep step on both operands.
#include "common.hpp"
#include "lds_dma.hpp"

namespace pgk {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kThreads = 256;
constexpr int BK = 128;          // bytes of K per slab = one scale group
constexpr int kFmtE4M3 = 0;      // f8f6f4 operand format code of e4m3

template <int BM, int BN>
struct Shape {
  static constexpr int WM = 2, WN = 2;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int SM = TM / 32, SN = TN / 32;
  static constexpr int A_BYTES = BM * BK;
  static constexpr int B_BYTES = BK * BN;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE + 16;
  static constexpr int A_INSTR = A_BYTES / 1024 / 4;
  static constexpr int B_INSTR = B_BYTES / 1024 / 4;
  static constexpr int B_ROWS_PER_INSTR = 1024 / BN;
  static constexpr int B_CPR = BN / 16;
  static_assert(SM <= 4 && SN <= 4, "scale bytes of at most 4 sub-tiles per register");
};

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS banks: 64 x 4 bytes; ds_read_b128 is served 16 lanes at a time,
// ds_read_b64 (and its transposing form) 32 lanes at a time.
// A rows are 128 bytes: the operand read touches 16 consecutive rows at one
// chunk, spread over 16 slots of a 256-byte window by XOR-ing (row >> 1).
__device__ __forceinline__ int swz_a(int row, int c) { return c ^ ((row >> 1) & 7); }
// B rows are BN bytes: a transposing read of 32 lanes touches 8 consecutive
// rows x 2 adjacent chunks.
template <int BN>
__device__ __forceinline__ int swz_b(int k, int c) {
  return BN >= 256 ? (c ^ (2 * (k & 7))) : (c ^ (k & 6));
}

template <int OPSEL_A, int OPSEL_B>
__device__ __forceinline__ f32x16 mfma_scaled(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFmtE4M3, kFmtE4M3, OPSEL_A, sa,
                                                         OPSEL_B, sb);
}

template <int BM, int BN, bool WITNESS>
__global__ void __launch_bounds__(kThreads) gemm_fp8_kernel(GemmParams P) {
  using S = Shape<BM, BN>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  int* s_tile = reinterpret_cast<int*>(smem + 2 * S::STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN;
  const int wn = wave % S::WN;
  const int prog = blockIdx.x;
  const int M = P.M, N = P.N, K = P.K;
  const unsigned char* __restrict__ A = static_cast<const unsigned char*>(P.A);
  const unsigned char* __restrict__ B = static_cast<const unsigned char*>(P.B);

  Walker walker(P.s, prog);
  long long t_start = 0;
  if (WITNESS && tid == 0) t_start = wall_ticks();

  // A: instruction q covers rows 8q .. 8q+7; lane p -> row 8q + p/8, LDS
  // chunk p%8, global chunk swz_a(row, p%8).
  auto a_row = [&](int q) { return q * 8 + (lane >> 3); };
  auto a_chunk = [&](int q) { return swz_a(a_row(q), lane & 7); };
  // B: instruction q covers rows R*q ..; lane p -> row R*q + p/CPR, LDS chunk
  // p%CPR, global chunk swz_b(row, p%CPR).
  auto b_row = [&](int q) { return q * S::B_ROWS_PER_INSTR + lane / S::B_CPR; };
  auto b_chunk = [&](int q) { return swz_b<BN>(b_row(q), lane % S::B_CPR); };

  // LDS read offsets.  A: lane l, sub-tile sm, step ks reads row
  // wm*TM + sm*32 + l%32, bytes ks*64 + (l/32)*32 .. +31 (two chunks).
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  unsigned rd_a[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = wm * S::TM + l32;
      const int c = swz_a(row, ks * 4 + hi * 2 + h);
      rd_a[ks][h] = (unsigned)(row * BK + c * 16);
    }
  // B^T: 16-lane group g, lane i -> row K0 + i/2, columns N0 + 8*(i%2);
  // N0 = wn*TN + sn*32 + (g&1)*16, K0 = ks*64 + hi*32 + 8r (r = 0..3).
  unsigned rd_b[S::SN];
  {
    const int g = lane >> 4, i16 = lane & 15, h = i16 & 1, e = i16 >> 1;
#pragma unroll
    for (int sn = 0; sn < S::SN; ++sn) {
      const int n = wn * S::TN + sn * 32 + (g & 1) * 16 + 8 * h;
      const int krow = hi * 32 + e;  // + ks*64 + 8r: multiples of 8 keep (row & 7) = e
      const int c = swz_b<BN>(krow, n >> 4);
      rd_b[sn] = (unsigned)(S::A_BYTES + krow * BN + c * 16 + (n & 15));
    }
  }

  // Scales of the slab: lane bytes for its sub-tile rows (opsel picks one).
  int sa_reg = 0, sb_reg = 0;      // current slab
  int sa_nxt = 0, sb_nxt = 0;      // prefetched for the next slab
  auto sload = [&](int m0, int n0, int k0, int& sa_out, int& sb_out) {
    const int grp = k0 / BK;
    const auto rSA = rsrc(P.sa + (size_t)grp * M, (unsigned)M);
    const auto rSB = rsrc(P.sb + (size_t)grp * N, (unsigned)N);
    unsigned va = 0, vb = 0;
#pragma unroll
    for (int s = 0; s < S::SM; ++s) {
      const int m = m0 + wm * S::TM + s * 32 + l32;
      va |= (unsigned)__builtin_amdgcn_raw_buffer_load_b8(rSA, m < M ? (unsigned)m : kOob, 0, 0) << (8 * s);
    }
#pragma unroll
    for (int s = 0; s < S::SN; ++s) {
      const int n = n0 + wn * S::TN + s * 32 + l32;
      vb |= (unsigned)__builtin_amdgcn_raw_buffer_load_b8(rSB, n < N ? (unsigned)n : kOob, 0, 0) << (8 * s);
    }
    sa_out = (int)va;
    sb_out = (int)vb;
  };

  auto gload = [&](int st, int m0, int n0, int k0) {
    unsigned char* sbase = smem + st * S::STAGE;
    const int rows = (M - m0) < BM ? (M - m0) : BM;
    const rsrc_words_t rA = rsrc_words(A + (size_t)m0 * K + k0, (unsigned)(rows * K - k0));
    const rsrc_words_t rB = rsrc_words(B + (size_t)k0 * N + n0, (unsigned)(BK * N - n0));
    const bool b_full = n0 + BN <= N;
#pragma unroll
    for (int i = 0; i < S::A_INSTR; ++i) {
      const int q = wave * S::A_INSTR + i;
      load_lds16(rA, sbase + q * 1024, (unsigned)a_row(q) * (unsigned)K + (unsigned)a_chunk(q) * 16u);
    }
#pragma unroll
    for (int i = 0; i < S::B_INSTR; ++i) {
      const int q = wave * S::B_INSTR + i;
      const int c = b_chunk(q);
      unsigned off = (unsigned)b_row(q) * (unsigned)N + (unsigned)c * 16u;
      if (!b_full && n0 + c * 16 >= N) off = kOob;
      load_lds16(rB, sbase + S::A_BYTES + q * 1024, off);
    }
  };

  f32x16 acc[S::SN][S::SM];

  auto compute = [&](int st) {
    const unsigned char* sbase = smem + st * S::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 bf[S::SN], af[S::SM];
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn) {
        const unsigned char* p = sbase + rd_b[sn] + ks * 64 * BN;
        i32x2 r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + q * 8 * BN));
        bf[sn] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
      }
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(sbase + rd_a[ks][0] + sm * 32 * BK);
        const i32x4 hh = *reinterpret_cast<const i32x4*>(sbase + rd_a[ks][1] + sm * 32 * BK);
        af[sm] = i32x8{lo[0], lo[1], lo[2], lo[3], hh[0], hh[1], hh[2], hh[3]};
      }
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn) {
#pragma unroll
        for (int sm = 0; sm < S::SM; ++sm) {
          // opsel selects the scale byte of sub-tile sn (B^T rows) / sm (A rows)
#define PGK_MFMA_CASE(a_, b_) \
  if (sn == a_ && sm == b_) acc[sn][sm] = mfma_scaled<a_, b_>(bf[sn], af[sm], acc[sn][sm], sb_reg, sa_reg);
          PGK_MFMA_CASE(0, 0) PGK_MFMA_CASE(0, 1) PGK_MFMA_CASE(0, 2) PGK_MFMA_CASE(0, 3)
          PGK_MFMA_CASE(1, 0) PGK_MFMA_CASE(1, 1) PGK_MFMA_CASE(1, 2) PGK_MFMA_CASE(1, 3)
          PGK_MFMA_CASE(2, 0) PGK_MFMA_CASE(2, 1) PGK_MFMA_CASE(2, 2) PGK_MFMA_CASE(2, 3)
          PGK_MFMA_CASE(3, 0) PGK_MFMA_CASE(3, 1) PGK_MFMA_CASE(3, 2) PGK_MFMA_CASE(3, 3)
#undef PGK_MFMA_CASE
        }
      }
    }
  };

  auto epilogue = [&](int m0, int n0) {
    const int rows = (M - m0) < BM ? (M - m0) : BM;
    const auto rC = rsrc(static_cast<unsigned char*>(P.C) + ((size_t)m0 * N + n0) * 2,
                         (unsigned)((size_t)rows * N - n0) * 2u);
    const int r0 = wm * S::TM + l32;
    const int c0 = wn * S::TN + 4 * hi;
    const unsigned eb = (unsigned)(r0 * N + c0) * 2u;
    const unsigned rstep = 32u * (unsigned)N * 2u;
    const int ncols = N - n0;
#pragma unroll
    for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cc = sn * 32 + 8 * g;
          const unsigned off = (c0 + cc < ncols) ? eb + sm * rstep + (unsigned)cc * 2u : kOob;
          const f32x16& a = acc[sn][sm];
          const u32x2 v = u32x2{pack_bf16x2(a[4 * g], a[4 * g + 1]),
                                pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
          __builtin_amdgcn_raw_buffer_store_b64(v, rC, off, 0, 0);
        }
  };

  const int nk = K / BK;
  if (tid == 0) s_tile[0] = walker.first();
  __syncthreads();
  int tile = __builtin_amdgcn_readfirstlane(s_tile[0]);
  int stage = 0;
  int it = 0;
  if (tile >= 0) {
    int pm, pn;
    walker.tile_coords(tile, pm, pn);
    gload(0, pm * BM, pn * BN, 0);
    sload(pm * BM, pn * BN, 0, sa_nxt, sb_nxt);
  }
  wait_vm0();
  slab_barrier();

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
      if (P.s.straggler_program == prog) spin_ns(P.s.straggler_ns, P.s.wall_khz);
    }
#pragma unroll
    for (int sn = 0; sn < S::SN; ++sn)
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[sn][sm][e] = 0.0f;

    const int slot = (it + 1) & 1;
    if (nk == 1 && tid == 0) s_tile[slot] = walker.next(tile);
    for (int kb = 0; kb + 1 < nk; ++kb) {
      if (kb == nk - 2 && tid == 0) s_tile[slot] = walker.next(tile);
      sa_reg = sa_nxt;
      sb_reg = sb_nxt;
      gload(stage ^ 1, m0, n0, (kb + 1) * BK);
      sload(m0, n0, (kb + 1) * BK, sa_nxt, sb_nxt);
      compute(stage);
      wait_vm0();
      slab_barrier();
      stage ^= 1;
    }
    sa_reg = sa_nxt;
    sb_reg = sb_nxt;
    int next = -1;
    if (nk >= 2) {
      next = __builtin_amdgcn_readfirstlane(s_tile[slot]);
      if (next >= 0) {
        int qm, qn;
        walker.tile_coords(next, qm, qn);
        gload(stage ^ 1, qm * BM, qn * BN, 0);
        sload(qm * BM, qn * BN, 0, sa_nxt, sb_nxt);
      }
    }
    compute(stage);
    wait_vm0();
    slab_barrier();
    stage ^= 1;
    epilogue(m0, n0);
    if (nk == 1) {
      next = __builtin_amdgcn_readfirstlane(s_tile[slot]);
      if (next >= 0) {
        int qm, qn;
        walker.tile_coords(next, qm, qn);
        gload(stage, qm * BM, qn * BN, 0);
        sload(qm * BM, qn * BN, 0, sa_nxt, sb_nxt);
      }
      wait_vm0();
      slab_barrier();
    }
    tile = next;
    ++it;
  }

  if (WITNESS && tid == 0) {
    P.w.t_start[prog] = t_start;
    P.w.t_end[prog] = wall_ticks();
    P.w.hw_id[prog] = hw_placement();
    P.w.n_tiles[prog] = it;
  }
}

template <int BM, int BN, bool WITNESS>
hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  using S = Shape<BM, BN>;
  auto kern = gemm_fp8_kernel<BM, BN, WITNESS>;
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

}  // namespace

bool gemm_fp8_tile_supported(int bm, int bn, int bk) {
  return bk == 128 && ((bm == 256 && bn == 256) || (bm == 128 && bn == 128));
}

// Shapes the kernel handles: K a multiple of 128 (checked by the caller), N a
// multiple of 16 (16-byte rows of B and C chunks), offsets within 32 bits.
bool gemm_fp8_eligible(int bm, long long N, long long K) {
  return N % 16 == 0 && (long long)bm * K < (1LL << 31) && 128LL * N < (1LL << 31) &&
         (long long)bm * N * 2 < (1LL << 31);
}

hipError_t launch_gemm_fp8(const GemmParams& p, int bm, int bn, int bk, bool vec, bool witness,
                           hipStream_t stream) {
  if (!vec || bk != 128) return hipErrorInvalidValue;
  if (bm == 256 && bn == 256)
    return witness ? launch_one<256, 256, true>(p, stream) : launch_one<256, 256, false>(p, stream);
  if (bm == 128 && bn == 128)
    return witness ? launch_one<128, 128, true>(p, stream) : launch_one<128, 128, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pgk
