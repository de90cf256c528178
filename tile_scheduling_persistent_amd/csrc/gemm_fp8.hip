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
// Data movement as in gemm_bf16_lds.hip: a ring of NST LDS stages of
// 128-deep slabs filled by hand-issued buffer_load ... lds (gemm_device.hpp),
// the loads of slab g + NST - 1 spread over the MFMAs of one slab period,
// the next step's fragment reads after each MFMA.  The slab barrier sits
// between the two 64-deep steps of a slab: after it, the previous slab's
// second step (fragments already in registers) covers the latency of the
// new slab's first reads.  The scale bytes of a slab travel
// with it: byte-sized direct loads put each row's (column's) scale byte in
// its own LDS dword of the stage, read back after the barrier.  Two stages
// suit the MFMA-bound square tiles; a deeper ring keeps more bytes in
// flight per CU where the kernel waits on HBM (few rows, long K).  A ([m][k], 128-byte
// rows) and B ([k][n]) are chunk-swizzled against LDS bank conflicts
// (swz_a, swz_b); A operands by ds_read_b128, B^T operands by
// ds_read_b64_tr_b8 (within a 16-lane group, lane i points at row
// K0 + i/2, columns N0 + 8*(i%2) .. +7, and lane j receives rows K0 .. K0+7
// of column N0 + j).  Lane l of the MFMA owns logical K positions
// 32*(l/32) .. +31 of each 64-deep step on both operands.
#include "common.hpp"
#include "gemm_device.hpp"

namespace pgk {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kThreads = 256;
constexpr int BK = 128;          // bytes of K per slab = one scale group
constexpr int kFmtE4M3 = 0;      // f8f6f4 operand format code of e4m3

template <int BM, int BN, int NST_>
struct Shape {
  static constexpr int NST = NST_;
  // Waves: 2 x 2 on square tiles; 1 x 4 on wide ones (128 x 256), where each
  // wave then reads every B^T byte of its columns once per tile and A (the
  // plain ds_read_b128 operand) four times, for the same LDS bytes as 2 x 2
  // in 16 reads per step instead of 20, half of them transposing instead of
  // four fifths.
  static constexpr int WM = BM < BN ? 1 : 2, WN = 4 / WM;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int SM = TM / 32, SN = TN / 32;
  static constexpr int A_BYTES = BM * BK;
  static constexpr int B_BYTES = BK * BN;
  // scale bytes: each wave loads those of its own TM rows / TN columns, 64
  // per byte-sized direct load, one LDS dword each
  static constexpr int SC_A = TM / 64, SC_B = TN / 64;
  static constexpr int NSC = SC_A + SC_B;
  static constexpr int SC_BYTES = 4 * NSC * 256;
  static constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  static constexpr int LDS_BYTES = NST * STAGE + 16;  // + first tile, next tile [2]
  static_assert(TM % 64 == 0 && TN % 64 == 0, "whole byte-load groups per wave");
  static_assert(NST >= 2 && NST <= 4, "LDS ring of two to four stages");
  static constexpr int A_INSTR = A_BYTES / 1024 / 4;
  static constexpr int B_INSTR = B_BYTES / 1024 / 4;
  static constexpr int B_ROWS_PER_INSTR = 1024 / BN;
  static constexpr int B_CPR = BN / 16;
  static_assert(SM <= 4 && SN <= 4, "scale bytes of at most 4 sub-tiles per register");
};

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

// GRP: several GEMMs in one launch (virtual tile ids shared by prefix sums,
// P.gp[g] from tile0 on); the loader and the matrix cores each look up the
// problem of their tile (operands, scales, sizes, slab count, output).
// SK: stream-K.  The program walks the segments (tile, first slab, end slab)
// of its stream-K run; a segment that does not cover its tile leaves fp32
// partial sums in the program's workspace slot, summed and stored by the
// fix-up kernel after this launch (the same one as the bf16 path's).
template <int BM, int BN, int NST, bool WITNESS, bool GRP, bool SK = false>
__global__ void __launch_bounds__(kThreads) gemm_fp8_kernel(GemmParams P) {
  using S = Shape<BM, BN, NST>;
  static_assert(!(SK && (GRP || WITNESS)), "stream-K runs one problem, without the witness");
  constexpr int NA = S::A_INSTR, NB = S::B_INSTR, NO = NA + NB;  // operand loads per wave per slab
  constexpr int NL = NO + S::NSC;                                // all loads per wave per slab
  constexpr int NMF = S::SN * S::SM;                             // MFMAs per 64-deep step
  constexpr int NRD = 4 * S::SN + 2 * S::SM;                     // LDS reads per step
  // The operand loads of a slab are spread over the first SPREAD MFMA
  // positions of its period (load d after position d*SPREAD/NO), one at a
  // time rather than a burst; its few scale-byte loads go out right after the
  // loader's bookkeeping.
  constexpr int SPREAD_W = 3 * NMF / 2 > NO ? 3 * NMF / 2 : NO;
  constexpr int SPREAD = SPREAD_W < 2 * NMF ? SPREAD_W : 2 * NMF;
  static_assert(SPREAD >= NO, "one operand load per MFMA at most");

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  int* s_first = reinterpret_cast<int*>(smem + NST * S::STAGE);
  int* s_next = s_first + 1;  // [2]: the loader's next tile, double-buffered by claim parity

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN;
  const int wn = wave % S::WN;
  const int prog = pgs::program_of(blockIdx.x, P.s.G, P.s.X, P.s.xcd_major);
  // The loader tile's problem and the matrix cores' tile's problem (one
  // problem unless GRP).
  int Ml = P.M, Nl = P.N, Kl = P.K;
  const unsigned char* Al = static_cast<const unsigned char*>(P.A);
  const unsigned char* Bl = static_cast<const unsigned char*>(P.B);
  const uint8_t* SAl = P.sa;
  const uint8_t* SBl = P.sb;
  int Mc = P.M, Nc = P.N;
  void* Cc = P.C;

  Walker walker(P.s, prog);
  if (WITNESS) walker.claim_row = P.w.claims + (size_t)prog * kMaxStealCounters;
  long long t_start = 0, c_start = 0;
  if (WITNESS && tid == 0) {
    t_start = wall_ticks();
    c_start = shader_cycles();
  }

  // Global -> LDS offsets.  A: instruction q covers rows 8q .. 8q+7; lane p
  // -> row 8q + p/8, LDS chunk p%8, global chunk swz_a(row, p%8).  B:
  // instruction q covers rows R*q ..; lane p -> row R*q + p/CPR, LDS chunk
  // p%CPR, global chunk swz_b(row, p%CPR).
  unsigned aoff[NA], boff[NB];
  int bchk[NB];
  // row strides K (A) and N (B), in bytes
  auto lane_offsets = [&](int Kx, int Nx) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = (wave * NA + i) * 8 + (lane >> 3);
      aoff[i] = (unsigned)row * (unsigned)Kx + (unsigned)swz_a(row, lane & 7) * 16u;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int row = (wave * NB + i) * S::B_ROWS_PER_INSTR + lane / S::B_CPR;
      bchk[i] = swz_b<BN>(row, lane % S::B_CPR);
      boff[i] = (unsigned)row * (unsigned)Nx + (unsigned)bchk[i] * 16u;
    }
  };
  lane_offsets(Kl, Nl);
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

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

  // Problem of virtual tile v (GRP): the last one whose first id is <= v,
  // selected with constant indices.
  auto problem_of = [&](int v) {
    GemmProblem pr = P.gp[0];
#pragma unroll
    for (int q = 1; q < kMaxGemmProblems; ++q)
      if (q < P.ngemm && v >= P.gp[q].tile0) pr = P.gp[q];
    return pr;
  };

  auto coords = [&](int v, int& m0, int& n0) {
    int pm, pn;
    if (GRP) {
      const GemmProblem pr = problem_of(v);
      pgs::decode(P.s.kind, v - pr.tile0, pr.npm, pr.npn, P.s.gs, pm, pn);
    } else {
      walker.tile_coords(v, pm, pn);
    }
    m0 = pm * BM;
    n0 = pn * BN;
  };

  int nkl = Kl / BK;  // slabs of the loader's tile

  // ---- loader state ----
  int lt = -1, lk = 0;      // loader: tile, next slab
  int lke = nkl;            // loader: end slab of its segment
  // Tiles the loader moved on to that the matrix cores have not reached: the
  // loader runs NST - 1 slabs ahead, so with one slab per tile that many can
  // wait (oldest first).
  int pend[NST - 1];
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) pend[i] = -1;
  int claims = 0;           // loader tile changes so far
  int lm0 = 0, ln0 = 0;     // loader tile origin
  rsrc_words_t rA, rB;      // resources of the slab being loaded
  unsigned long long a_ptr = 0, b_ptr = 0;  // the loader tile's A rows / B columns at k = 0
  unsigned a_rec = 0;                       // bytes of A from a_ptr to the tile's last row
  unsigned bo[NB];          // B offsets (column chunks past N pushed out of range)
  bool masked = true;       // bo holds masked offsets
  // scale byte offsets of the wave's rows / columns (64 per load, lane = row)
  unsigned soa[S::SC_A], sob[S::SC_B];
  rsrc_words_t rSA, rSB;    // scale rows of the slab being loaded

  // Stream-K segment walkers of this program: one for the loader, one for
  // the matrix cores (the same sequence, read at different times).
  pgs::SkWalker lw, cw;
  if (SK) {
    lw.init(prog, P.s.T, P.s.G, P.K / BK);
    cw.init(prog, P.s.T, P.s.G, P.K / BK);
  }

  // Pick the next slab for the loader (moving on to the next tile once the
  // current one is issued), set up its resources and load its scales;
  // without one the resources are empty and the loads read zeros into a
  // stage no one reads.
  // The loader moves on to slabs [kb, ke) of tile t (t >= 0; ke < 0: to the
  // end of the tile): per-tile bases, B offsets with column chunks past N
  // pushed out of range, scale byte offsets.
  auto begin_tile = [&](int t, int kb, int ke) {
    lt = t;
    lk = kb;
    if (GRP) {
      const GemmProblem pr = problem_of(t);
      Al = static_cast<const unsigned char*>(pr.A);
      Bl = static_cast<const unsigned char*>(pr.B);
      SAl = pr.sa;
      SBl = pr.sb;
      Ml = pr.M;
      Nl = pr.N;
      Kl = pr.K;
      nkl = Kl / BK;
      lane_offsets(Kl, Nl);
      masked = true;  // bo is rebuilt from the new offsets
    }
    lke = ke < 0 ? nkl : ke;
    coords(t, lm0, ln0);
    int rows = (Ml - lm0) < BM ? (Ml - lm0) : BM;
    rows = rows < 0 ? 0 : rows;  // never negative: an empty range reads zeros
    a_ptr = reinterpret_cast<unsigned long long>(Al + (size_t)lm0 * Kl);
    a_rec = (unsigned)(rows * Kl);
    b_ptr = reinterpret_cast<unsigned long long>(Bl + ln0);
    const bool edge = ln0 + BN > Nl;
    if (edge || masked) {
#pragma unroll
      for (int i = 0; i < NB; ++i) bo[i] = (ln0 + bchk[i] * 16 < Nl) ? boff[i] : kOob;
      masked = edge;
    }
#pragma unroll
    for (int i = 0; i < S::SC_A; ++i) {
      const int m = lm0 + wm * S::TM + i * 64 + lane;
      soa[i] = m < Ml ? (unsigned)m : kOob;
    }
#pragma unroll
    for (int i = 0; i < S::SC_B; ++i) {
      const int n = ln0 + wn * S::TN + i * 64 + lane;
      sob[i] = n < Nl ? (unsigned)n : kOob;
    }
  };

  auto prep = [&]() {
    // The loader state is the same in every lane; saying so keeps its
    // branches scalar.
    lt = __builtin_amdgcn_readfirstlane(lt);
    lk = __builtin_amdgcn_readfirstlane(lk);
    lke = __builtin_amdgcn_readfirstlane(lke);
    claims = __builtin_amdgcn_readfirstlane(claims);
    if (lt >= 0 && lk == lke) {
      lt = -1;
      if (SK) {
        int v, kb, ke, slot;
        if (lw.next(v, kb, ke, slot)) begin_tile(v, kb, ke);
      } else {
        const int t = __builtin_amdgcn_readfirstlane(s_next[claims & 1]);
        ++claims;
        if (t >= 0) {
          bool queued = false;  // into the first free entry (entries fill from 0)
#pragma unroll
          for (int i = 0; i < NST - 1; ++i)
            if (!queued && pend[i] < 0) {
              pend[i] = t;
              queued = true;
            }
          begin_tile(t, 0, -1);
        }
      }
    }
    const int k0 = lk * BK;
    const bool load = lt >= 0;
    if (load) {
      ++lk;
      if (!SK && lk == lke && tid == 0) s_next[claims & 1] = walker.next(lt);
    }
    rA = rsrc_words_u64(a_ptr + (unsigned long long)k0, load ? a_rec - (unsigned)k0 : 0u);
    rB = rsrc_words_u64(b_ptr + (unsigned long long)k0 * (unsigned long long)Nl,
                        load ? (unsigned)(BK * Nl - ln0) : 0u);
    const int grp = k0 / BK;
    rSA = rsrc_words_u64(reinterpret_cast<unsigned long long>(SAl + (size_t)grp * Ml), load ? (unsigned)Ml : 0u);
    rSB = rsrc_words_u64(reinterpret_cast<unsigned long long>(SBl + (size_t)grp * Nl), load ? (unsigned)Nl : 0u);
  };

  // LDS dwords of this wave's scale bytes in a stage: A rows, then B columns.
  const unsigned sc_off = (unsigned)(S::A_BYTES + S::B_BYTES + wave * S::NSC * 256);

  // Load d of the prepared slab into stage st: operand chunks, then the
  // wave's scale bytes.
  auto dma = [&](int st, int d) {
    const unsigned sb = lds0 + (unsigned)(st * S::STAGE);
    if (d < NA)
      load_lds16(rA, sb + (unsigned)((wave * NA + d) * 1024), aoff[d]);
    else if (d < NO)
      load_lds16(rB, sb + (unsigned)(S::A_BYTES + (wave * NB + d - NA) * 1024), bo[d - NA]);
    else if (d < NO + S::SC_A)
      load_lds_u8(rSA, sb + sc_off + (unsigned)((d - NO) * 256), soa[d - NO]);
    else
      load_lds_u8(rSB, sb + sc_off + (unsigned)((d - NO) * 256), sob[d - NO - S::SC_A]);
  };

  f32x16 acc[S::SN][S::SM];
  // Operand fragments, double-buffered by step: B^T blocks as four 8-byte
  // transposed pieces, A blocks as two 16-byte pieces.
  i32x2 bq[2][S::SN][4];
  i32x4 aq[2][S::SM][2];
  int sa_reg = 0, sb_reg = 0;  // scales of the slab on the matrix cores

  // LDS read r of step ks into slot: B^T block 0 first, then the A blocks,
  // then the other B^T blocks (the order the MFMAs consume them).
  auto read = [&](int st, int ks, int slot, int r) {
    const unsigned char* sbase = smem + st * S::STAGE;
    if (r >= 4 && r < 4 + 2 * S::SM) {
      const int sm = (r - 4) >> 1, h = (r - 4) & 1;
      aq[slot][sm][h] = *reinterpret_cast<const i32x4*>(sbase + rd_a[ks][h] + sm * 32 * BK);
    } else {
      const int b = r < 4 ? r : r - 2 * S::SM;
      const int sn = b >> 2, q = b & 3;
      const unsigned char* p = sbase + rd_b[sn] + ks * 64 * BN + q * 8 * BN;
      bq[slot][sn][q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
    }
  };

  auto mfma = [&](int slot, int j) {
    const int sn = j / S::SM, sm = j % S::SM;
    const i32x2* b4 = bq[slot][sn];
    const i32x8 bf = i32x8{b4[0][0], b4[0][1], b4[1][0], b4[1][1], b4[2][0], b4[2][1], b4[3][0], b4[3][1]};
    const i32x4* a2 = aq[slot][sm];
    const i32x8 af = i32x8{a2[0][0], a2[0][1], a2[0][2], a2[0][3], a2[1][0], a2[1][1], a2[1][2], a2[1][3]};
    // opsel selects the scale byte of sub-tile sn (B^T rows) / sm (A rows)
#define PGK_MFMA_CASE(a_, b_) \
    if (sn == a_ && sm == b_) acc[sn][sm] = mfma_scaled<a_, b_>(bf, af, acc[sn][sm], sb_reg, sa_reg);
    PGK_MFMA_CASE(0, 0) PGK_MFMA_CASE(0, 1) PGK_MFMA_CASE(0, 2) PGK_MFMA_CASE(0, 3)
    PGK_MFMA_CASE(1, 0) PGK_MFMA_CASE(1, 1) PGK_MFMA_CASE(1, 2) PGK_MFMA_CASE(1, 3)
    PGK_MFMA_CASE(2, 0) PGK_MFMA_CASE(2, 1) PGK_MFMA_CASE(2, 2) PGK_MFMA_CASE(2, 3)
    PGK_MFMA_CASE(3, 0) PGK_MFMA_CASE(3, 1) PGK_MFMA_CASE(3, 2) PGK_MFMA_CASE(3, 3)
#undef PGK_MFMA_CASE
  };

  auto epilogue = [&](int m0, int n0) {
    const int N = Nc;
    int rows = (Mc - m0) < BM ? (Mc - m0) : BM;
    rows = rows < 0 ? 0 : rows;  // never negative: an empty range drops the stores
    const auto rC = rsrc(static_cast<unsigned char*>(Cc) + ((size_t)m0 * N + n0) * 2,
                         (unsigned)((size_t)rows * N - n0) * 2u);
    const int r0 = wm * S::TM + l32;
    const unsigned eb = (unsigned)(r0 * N) * 2u;
    const unsigned rstep = 32u * (unsigned)N * 2u;
    const int ncols = N - n0;
#pragma unroll
    for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn)
        store_block_bf16(acc[sn][sm], rC, eb + sm * rstep, wn * S::TN + sn * 32, ncols, hi);
  };

  // Stream-K: the accumulators of a partial segment, fp32, into slot `slot`
  // of this program's workspace ([BM][BN], tile-relative).
  auto store_partial = [&](int slot) {
    float* wsb = P.ws + ((size_t)prog * 2 + slot) * (size_t)(BM * BN);
    const int r0 = wm * S::TM + l32;
    const int c0 = wn * S::TN + 4 * hi;
#pragma unroll
    for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[sn][sm];
          *reinterpret_cast<f32x4*>(wsb + (r0 + sm * 32) * BN + c0 + sn * 32 + 8 * q) =
              f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        }
  };

  int ct = -1;               // tile on the matrix cores
  int cnk = P.K / BK;        // its slab count
  int cslot = -1;            // its partial-sum slot (stream-K)
  if (SK) {
    int kb, ke;
    if (cw.next(ct, kb, ke, cslot)) cnk = ke - kb;
  } else {
    if (tid == 0) s_first[0] = walker.first();
    __syncthreads();
    ct = __builtin_amdgcn_readfirstlane(s_first[0]);
  }
  if (ct >= 0) {
    if (SK) {
      int v, kb, ke, slot;
      lw.next(v, kb, ke, slot);
      begin_tile(v, kb, ke);
    } else {
      begin_tile(ct, 0, -1);
    }
    // slabs 0 .. NST-2 into stages 0 .. NST-2 (a barrier between preps: a
    // claim thread 0 stores in one is read by every wave in the next)
#pragma unroll
    for (int j = 0; j < NST - 1; ++j) {
      if (j > 0) slab_barrier();
      prep();
#pragma unroll
      for (int d = 0; d < NL; ++d) dma(j, d);
    }
  }

  int g = 0;   // slabs computed so far
  int it = 0;  // tiles finished
  int m0 = 0, n0 = 0;  // origin of tile ct
  // The matrix cores move on to tile ct: its origin and (GRP) its problem's
  // output and slab count.
  auto compute_tile = [&]() {
    coords(ct, m0, n0);
    if (GRP) {
      const GemmProblem pr = problem_of(ct);
      Mc = pr.M;
      Nc = pr.N;
      Cc = pr.C;
      cnk = pr.K / BK;
    }
  };
  if (ct >= 0) compute_tile();
  while (ct >= 0) {
    if (tid == 0) {
      if (WITNESS) {
        atomicAdd(P.w.visits + ct, 1);
        P.w.owner[ct] = prog;
        P.w.order[ct] = it;
      }
      if (is_straggler(P.s, prog)) spin_ns(P.s.straggler_ns, P.s.wall_khz);
    }
#pragma unroll
    for (int sn = 0; sn < S::SN; ++sn)
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[sn][sm][e] = 0.0f;
    // One period per slab g: barrier, then step 1 of slab g-1 (fragments in
    // slot 1, scales of g-1) while step 0 of slab g is read into slot 0, then
    // step 0 of slab g while its step 1 is read into slot 1.  The barrier thus
    // sits between the two steps of a slab, and the first MFMAs after it use
    // fragments already in registers: the latency of the new slab's first
    // reads hides under the old slab's second step instead of stalling the
    // matrix cores.  The tile's first slab (peeled off the loop) has no
    // previous step to overlap; its last slab's step 1 runs after the loop.
    //
    // Slab g (operands and scale bytes) landed once this wave's loads of it
    // are done (the loads of the NST - 2 slabs after it may still be in
    // flight) and every wave has passed the barrier.  Every wave has also
    // finished its LDS reads of slab g-1 (lgkmcnt(0) before the barrier; its
    // step 1 is in registers), which frees that stage for the loads of slab
    // g + NST - 1.
    auto slab_start = [&](unsigned (&sraw)[S::SM + S::SN]) {
      wait_vm<(NST - 2) * NL>();
      slab_barrier();
      const unsigned char* scb = smem + (g % NST) * S::STAGE + sc_off;
#pragma unroll
      for (int s = 0; s < S::SM; ++s)
        sraw[s] = *reinterpret_cast<const unsigned*>(scb + (s * 32 + l32) * 4);
#pragma unroll
      for (int s = 0; s < S::SN; ++s)
        sraw[S::SM + s] = *reinterpret_cast<const unsigned*>(scb + S::SC_A * 256 + (s * 32 + l32) * 4);
      __builtin_amdgcn_sched_barrier(0);
    };
    // A slab's scale bytes packed for opsel: byte s of the A word is the
    // scale of sub-tile sm = s, likewise for B.
    auto pack_scales = [&](const unsigned (&sraw)[S::SM + S::SN], int& va_out, int& vb_out) {
      unsigned va = 0, vb = 0;
#pragma unroll
      for (int s = 0; s < S::SM; ++s) va |= (sraw[s] & 0xffu) << (8 * s);
#pragma unroll
      for (int s = 0; s < S::SN; ++s) vb |= (sraw[S::SM + s] & 0xffu) << (8 * s);
      va_out = (int)va;
      vb_out = (int)vb;
    };
    // Step 0 of slab g with its step-1 reads and the rest of the loads.
    auto step0_period = [&](int st, int st_dma) {
#pragma unroll
      for (int j = 0; j < NMF; ++j) {
        mfma(0, j);
#pragma unroll
        for (int r = j * NRD / NMF; r < (j + 1) * NRD / NMF; ++r) read(st, 1, 1, r);
#pragma unroll
        for (int d = 0; d < NO; ++d)
          if (d * SPREAD / NO == NMF + j) dma(st_dma, d);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++g;
    };
    {
      // first slab of the tile: its step-0 reads, the loader's bookkeeping
      // under their latency, then the loads of the first MFMA positions
      unsigned sraw[S::SM + S::SN];
      slab_start(sraw);
      const int st = g % NST;
      const int st_dma = st == 0 ? NST - 1 : st - 1;
#pragma unroll
      for (int r = 0; r < NRD; ++r) read(st, 0, 0, r);
      __builtin_amdgcn_sched_barrier(0);
      prep();  // slab g + NST - 1
#pragma unroll
      for (int d = NO; d < NL; ++d) dma(st_dma, d);
#pragma unroll
      for (int d = 0; d < NO; ++d)
        if (d * SPREAD / NO < NMF) dma(st_dma, d);
      pack_scales(sraw, sa_reg, sb_reg);
      __builtin_amdgcn_sched_barrier(0);
      step0_period(st, st_dma);
    }
    for (int ck = 1; ck < cnk; ++ck) {
      unsigned sraw[S::SM + S::SN];
      slab_start(sraw);
      const int st = g % NST;
      const int st_dma = st == 0 ? NST - 1 : st - 1;
      // step 1 of slab g-1 while step 0 of slab g is read; the loader's
      // bookkeeping after its first MFMA
      mfma(1, 0);
#pragma unroll
      for (int r = 0; r < NRD / NMF; ++r) read(st, 0, 0, r);
      __builtin_amdgcn_sched_barrier(0);
      prep();  // slab g + NST - 1
#pragma unroll
      for (int d = NO; d < NL; ++d) dma(st_dma, d);
#pragma unroll
      for (int d = 0; d < NO; ++d)
        if (d * SPREAD / NO == 0) dma(st_dma, d);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 1; j < NMF; ++j) {
        mfma(1, j);
#pragma unroll
        for (int r = j * NRD / NMF; r < (j + 1) * NRD / NMF; ++r) read(st, 0, 0, r);
#pragma unroll
        for (int d = 0; d < NO; ++d)
          if (d * SPREAD / NO == j) dma(st_dma, d);
        __builtin_amdgcn_sched_barrier(0);
      }
      pack_scales(sraw, sa_reg, sb_reg);
      __builtin_amdgcn_sched_barrier(0);
      step0_period(st, st_dma);
    }
    // step 1 of the tile's last slab, then the wait for its results (the
    // epilogue reads the accumulators with acc_read)
#pragma unroll
    for (int j = 0; j < NMF; ++j) {
      mfma(1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_results_ready();
    if (SK && cslot >= 0)
      store_partial(cslot);
    else
      epilogue(m0, n0);
    ++it;
    if (SK) {
      int kb, ke;
      ct = -1;
      if (cw.next(ct, kb, ke, cslot)) cnk = ke - kb;
    } else {
      ct = pend[0];
#pragma unroll
      for (int i = 0; i + 1 < NST - 1; ++i) pend[i] = pend[i + 1];
      pend[NST - 2] = -1;
    }
    if (ct >= 0) compute_tile();
  }

  if (WITNESS && tid == 0) {
    P.w.t_start[prog] = t_start;
    P.w.t_end[prog] = wall_ticks();
    P.w.cycles[prog] = shader_cycles() - c_start;
    P.w.hw_id[prog] = hw_placement();
    P.w.n_tiles[prog] = it;
  }
}

template <int BM, int BN, int NST, bool WITNESS, bool GRP = false, bool SK = false>
hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  using S = Shape<BM, BN, NST>;
  auto kern = gemm_fp8_kernel<BM, BN, NST, WITNESS, GRP, SK>;
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

template <int BM, int BN, int NST, bool GRP = false>
KernelInfo info_one() {
  using S = Shape<BM, BN, NST>;
  static const KernelInfo ki = {
      kThreads, S::LDS_BYTES,
      occupancy_of(reinterpret_cast<const void*>(gemm_fp8_kernel<BM, BN, NST, false, GRP>), kThreads,
                   S::LDS_BYTES)};
  return ki;
}

}  // namespace

// Built tiles and their LDS rings: 256x256 and 128x128 (two stages), 128x256
// (three stages: one program per CU with twice the B bytes of a 128x128
// program in flight per slab, for shapes with few rows).
bool gemm_fp8_tile_supported(int bm, int bn, int bk) {
  return bk == 128 && ((bm == 256 && bn == 256) || (bm == 128 && bn == 128) || (bm == 128 && bn == 256));
}

// Shapes the kernel handles: K a multiple of 128 (checked by the caller), N a
// multiple of 16 (16-byte rows of B and C chunks), offsets within 32 bits.
bool gemm_fp8_eligible(int bm, long long N, long long K) {
  return N % 16 == 0 && (long long)bm * K < (1LL << 31) && 128LL * N < (1LL << 31) &&
         (long long)bm * N * 2 < (1LL << 31);
}

KernelInfo info_gemm_fp8(int bm, int bn) {
  if (bm == 256 && bn == 256) return info_one<256, 256, 2>();
  if (bm == 128 && bn == 128) return info_one<128, 128, 2>();
  if (bm == 128 && bn == 256) return info_one<128, 256, 3>();
  return KernelInfo{0, 0, 0};
}

hipError_t launch_gemm_fp8(const GemmParams& p, int bm, int bn, int bk, bool vec, bool witness,
                           hipStream_t stream) {
  if (!vec || bk != 128) return hipErrorInvalidValue;
  if (bm == 256 && bn == 256)
    return witness ? launch_one<256, 256, 2, true>(p, stream) : launch_one<256, 256, 2, false>(p, stream);
  if (bm == 128 && bn == 128)
    return witness ? launch_one<128, 128, 2, true>(p, stream) : launch_one<128, 128, 2, false>(p, stream);
  if (bm == 128 && bn == 256)
    return witness ? launch_one<128, 256, 3, true>(p, stream) : launch_one<128, 256, 3, false>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_fp8_sk(const GemmParams& p, int bm, int bn, hipStream_t stream) {
  if (bm == 256 && bn == 256) return launch_one<256, 256, 2, false, false, true>(p, stream);
  if (bm == 128 && bn == 128) return launch_one<128, 128, 2, false, false, true>(p, stream);
  if (bm == 128 && bn == 256) return launch_one<128, 256, 3, false, false, true>(p, stream);
  return hipErrorInvalidValue;
}

KernelInfo info_gemm_fp8_grouped(int bm, int bn) {
  if (bm == 256 && bn == 256) return info_one<256, 256, 2, true>();
  if (bm == 128 && bn == 128) return info_one<128, 128, 2, true>();
  if (bm == 128 && bn == 256) return info_one<128, 256, 3, true>();
  return KernelInfo{0, 0, 0};
}

hipError_t launch_gemm_fp8_grouped(const GemmParams& p, int bm, int bn, bool witness, hipStream_t stream) {
  if (p.ngemm < 1 || p.ngemm > kMaxGemmProblems) return hipErrorInvalidValue;
  if (bm == 256 && bn == 256)
    return witness ? launch_one<256, 256, 2, true, true>(p, stream) : launch_one<256, 256, 2, false, true>(p, stream);
  if (bm == 128 && bn == 128)
    return witness ? launch_one<128, 128, 2, true, true>(p, stream) : launch_one<128, 128, 2, false, true>(p, stream);
  if (bm == 128 && bn == 256)
    return witness ? launch_one<128, 256, 3, true, true>(p, stream) : launch_one<128, 256, 3, false, true>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pgk
