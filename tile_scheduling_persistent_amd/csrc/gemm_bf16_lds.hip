// Persistent bf16 GEMM for gfx950, fast path (K and N multiples of 8,
// 16-byte aligned operands): C[M][N] = A[M][K] . B[K][N], fp32 accumulate.
//
// Same persistent tile loop and schedulers as gemm_bf16.hip ("Work Stealing
// Scheduler Kernel", tritonBLAS PR #65; "Implement persistent kernels",
// Helion PR #238).  What differs is how operands reach the matrix cores:
//  * Global -> LDS with buffer_load ... lds (16 bytes per lane, 1 KiB per
//    wave instruction): no staging registers, no VALU work.  The LDS side of
//    such a load is linear, so the bank swizzle is applied on the global side
//    (each lane fetches the chunk that belongs at its LDS position).
//  * Two LDS stages of 64-deep slabs: while the matrix cores work on slab g
//    the loads of slab g+1 fill the other stage, and the loader walks
//    straight on into the next tile of the schedule (the pipeline phase runs
//    on across tiles, like the scheduler's iteration counter of "[Feature]
//    Introduce tile scheduler", TileLang PR #2441).  The next tile is
//    claimed when the loader sets up the last slab of the current one.
//  * A slab is two 32-deep k-steps, run as four phases of half a k-step
//    each (one half of the B^T blocks).  One barrier per slab, after its
//    third phase: each wave has waited for its own loads of slab g+1 (vmcnt)
//    and finished every read of slab g, so after the barrier slab g+1 is
//    complete and slab g's stage is free.  The last phase then reads slab
//    g+1's first fragments and starts slab g+2's loads; the loads are issued
//    by hand and the barrier carries no memory fence (gemm_device.hpp), so
//    the compiler adds no wait for loads in flight before LDS reads.
//  * The issue order inside a phase is fixed by hand (scheduling barriers):
//    after each MFMA come its share of the fragment reads the next phase
//    needs and, in phases 0 and 3, a load, so LDS reads, global loads and
//    their latencies hide behind the MFMA pipeline instead of stalling the
//    wave in bursts; each load has at least two phases to land.  The
//    loader's bookkeeping (tile switch, claim, buffer resources) is scalar
//    pointer arithmetic except on edge slabs.
//  * A stays [m][k] in LDS; its 16-byte chunks are XOR-swizzled by the row
//    so that the ds_read_b128 operand reads hit distinct banks (see bf16_swz_a).
//  * B stays [k][n] in LDS, as it is in memory (chunk c of row k stored at
//    c ^ 4*(k & 3) ^ 2*((k >> 3) & 1), see swz_b16); the k-contiguous
//    operand the MFMA needs is produced by ds_read_b64_tr_b16: within each
//    16-lane group, lane i points at row K0 + i/4, columns N0 + 4*(i%4) ..
//    +3, and lane j receives rows K0 .. K0+3 of column N0 + j.  Two such
//    reads give a lane its 8 k-values; the four 16-lane groups take k rows
//    8g .. 8g+7 of the 32-deep step.
//  * Each wave owns a (BM/2) x (BN/2) sub-tile as 16x16 MFMA blocks
//    (v_mfma_f32_16x16x32_bf16) with the B^T block as the first operand, so
//    lane l holds row l % 16 of a block and its 4 accumulators are 4
//    consecutive columns of C (4*(l/16) .. +3).  Against 32x32x16 blocks
//    the 16x16x32 form moves half the fp32 accumulator bytes through the
//    register file per product; on this chip, whose clock is held down by
//    its power limit under these GEMMs, that buys clock: register-only MFMA
//    loops on random bf16 data ran 11% more flops at the same board power,
//    and this kernel 3-5% more TFLOP/s on normal(0,1) operands.
//  * Rows past M (A) and past K (B) read as zero through the buffer range
//    check; the K tail and columns past N are masked per lane, only on the
//    slabs / tiles that need it; C stores outside the matrix are dropped by
//    the range check or masked (no index wrapping; review of the
//    work-stealing kernel in tritonBLAS PR #65).
#include "common.hpp"
#include "gemm_device.hpp"

namespace pgk {
namespace {

// Physical chunk of logical chunk c in row k of B for the 16x16 fragment
// reads: 32 lanes of a transposing read touch rows k0..k0+3 and k0+8..k0+11
// at two adjacent chunks; bits 2-3 from k & 3 and bit 1 from bit 3 of k put
// those 16 chunks in 16 distinct slots of a 256-byte window.
__device__ __forceinline__ int swz_b16(int k, int c) { return c ^ (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;
constexpr int kAuxNonTemporal = 2;  // buffer store cache-policy bits: nt

template <int BM, int BN, int BK, int NST>
struct Shape {
  static constexpr int WM = 2, WN = 2;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int SM = TM / 16, SN = TN / 16;   // 16x16 MFMA blocks
  static constexpr int KK = BK / 32;                  // MFMA k-steps per slab
  static constexpr int A_ROW = BK * 2;                // bytes per LDS row of A
  static constexpr int A_BYTES = BM * A_ROW;          // one stage of A
  static constexpr int B_ROW = BN * 2;                // bytes per LDS row of B
  static constexpr int B_BYTES = BK * B_ROW;          // one stage of B
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NST * STAGE + 32;
  static constexpr int A_INSTR = A_BYTES / 1024 / 4;  // 1 KiB loads per wave per slab
  static constexpr int B_INSTR = B_BYTES / 1024 / 4;
  static constexpr int A_RPI = 1024 / A_ROW;          // A rows per load instruction
  static constexpr int A_CPR = A_ROW / 16;            // 16-byte chunks per A row
  static constexpr int B_RPI = 1024 / B_ROW;
  static constexpr int B_CPR = B_ROW / 16;
  static_assert(BK == 32 || BK == 64, "slab depth");
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && 1024 % B_ROW == 0, "slab splits into 1 KiB loads");
};

// SK: stream-K.  The program walks segments (tile, first slab, end slab)
// of its own stream-K run instead of whole tiles; a segment that does not
// cover its tile leaves fp32 partial sums in the program's workspace slot,
// summed and stored by the fix-up kernel after this launch.
// GRP: several GEMMs in one launch.  Their tiles share one virtual id space
// (problem g from P.gp[g].tile0 on); the loader and the matrix cores each
// look up the problem of their tile (operands, sizes, slab count) when they
// move on to it.
template <int BM, int BN, int BK, int NST, bool OUT_BF16, bool WITNESS, bool SK, bool GRP>
__global__ void __launch_bounds__(kThreads) gemm_bf16_lds_kernel(GemmParams P) {
  using S = Shape<BM, BN, BK, NST>;
  static_assert(NST == 2, "two LDS stages: the loads of slab g+1 run during slab g");
  static_assert(S::KK == 2 && S::SN % 2 == 0, "two 32-deep k-steps per slab, B blocks in two halves");
  constexpr int NA = S::A_INSTR, NB = S::B_INSTR, NL = NA + NB;  // loads per wave per slab
  constexpr int NMF = S::SN * S::SM;                             // MFMAs per k-step

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
  const unsigned short* Al = static_cast<const unsigned short*>(P.A);
  const unsigned short* Bl = static_cast<const unsigned short*>(P.B);
  int Mc = P.M, Nc = P.N;
  void* Cc = P.C;

  Walker walker(P.s, prog);
  if (WITNESS) walker.claim_row = P.w.claims + (size_t)prog * kMaxStealCounters;
  long long t_start = 0, c_start = 0;
  if (WITNESS && tid == 0) {
    t_start = wall_ticks();
    c_start = shader_cycles();
  }

  // ---- global -> LDS load offsets (per lane, relative to the slab bases) ----
  // A: instruction q covers rows RPI*q ..; lane p -> row RPI*q + p/CPR, LDS
  // chunk p%CPR, global chunk bf16_swz_a(row, p%CPR) (the swizzle is an
  // involution).  B likewise with bf16_swz_b.
  unsigned aoff[NA], boff[NB];
  int achk[NA], bchk[NB];
  // row strides K (A) and N (B), in elements
  auto lane_offsets = [&](int Kx, int Nx) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = wave * NA + i;
      const int row = q * S::A_RPI + lane / S::A_CPR;
      achk[i] = bf16_swz_a<BK>(row, lane % S::A_CPR);
      aoff[i] = (unsigned)row * (unsigned)Kx * 2u + (unsigned)achk[i] * 16u;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = wave * NB + i;
      const int row = q * S::B_RPI + lane / S::B_CPR;
      bchk[i] = swz_b16(row, lane % S::B_CPR);
      boff[i] = (unsigned)row * (unsigned)Nx * 2u + (unsigned)bchk[i] * 16u;
    }
  };
  lane_offsets(Kl, Nl);
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  // ---- LDS read offsets ----
  const int l16 = lane & 15;
  unsigned rd_a[S::KK];
#pragma unroll
  for (int kk = 0; kk < S::KK; ++kk) {
    const int row = wm * S::TM + l16;  // + sm*16: swizzle unchanged
    rd_a[kk] = (unsigned)(row * S::A_ROW + bf16_swz_a<BK>(row, kk * 4 + (lane >> 4)) * 16);
  }
  unsigned rd_b[S::SN];
  {
    const int g = lane >> 4, i16 = lane & 15, a = i16 & 3, e = i16 >> 2;
    const int krow = g * 8 + e;  // + kk*32 + h*4: k & 3 and bit 3 of k unchanged
#pragma unroll
    for (int sn = 0; sn < S::SN; ++sn) {
      const int n = wn * S::TN + sn * 16 + 4 * a;
      const int c = swz_b16(krow, n >> 3);
      rd_b[sn] = (unsigned)(S::A_BYTES + krow * S::B_ROW + c * 16 + 8 * (a & 1));
    }
  }

  // Problem of virtual tile v (GRP): the last one whose first id is <= v
  // (empty problems own no ids), selected with constant indices.
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

  const int nk = (P.K + BK - 1) / BK;

  // ---- loader state ----
  int lt = -1, lk = 0;      // loader: tile, next slab
  int lke = nk;             // loader: end slab of its segment
  // Tiles the loader moved on to that the matrix cores have not reached:
  // the loader runs two slabs ahead, so with one slab per tile two can wait.
  int pend0 = -1, pend1 = -1;
  int claims = 0;           // loader tile changes so far
  int lm0 = 0, ln0 = 0;     // loader tile origin
  rsrc_words_t rA, rB;      // resources of the slab being loaded
  unsigned long long a_ptr = 0, b_ptr = 0;  // the loader tile's A rows / B columns at k = 0
  unsigned a_rec = 0;                       // bytes of A from a_ptr to the tile's last row
  unsigned ao[NA], bo[NB];  // per-lane offsets (edge chunks pushed out of range)
  bool masked = true;       // ao / bo hold masked offsets

  // Stream-K segment walkers of this program: one for the loader, one for
  // the matrix cores (the same sequence, read at different times).
  pgs::SkWalker lw, cw;
  if (SK) {
    lw.init(prog, P.s.T, P.s.G, nk);
    cw.init(prog, P.s.T, P.s.G, nk);
  }

  // The loader moves on to slabs [kb, ke) of tile t (t >= 0; ke < 0: to
  // the end of the tile).
  auto begin_tile = [&](int t, int kb, int ke) {
    lt = t;
    lk = kb;
    if (GRP) {
      const GemmProblem pr = problem_of(t);
      Al = static_cast<const unsigned short*>(pr.A);
      Bl = static_cast<const unsigned short*>(pr.B);
      Ml = pr.M;
      Nl = pr.N;
      Kl = pr.K;
      lane_offsets(Kl, Nl);
      masked = true;  // ao / bo are rebuilt from the new offsets
    }
    lke = ke < 0 ? (Kl + BK - 1) / BK : ke;
    coords(t, lm0, ln0);
    int rows = (Ml - lm0) < BM ? (Ml - lm0) : BM;
    rows = rows < 0 ? 0 : rows;  // never negative: an empty range reads zeros
    a_ptr = reinterpret_cast<unsigned long long>(Al + (size_t)lm0 * Kl);
    a_rec = (unsigned)(rows * Kl) * 2u;
    b_ptr = reinterpret_cast<unsigned long long>(Bl + ln0);
  };

  // Pick the next slab for the loader (moving on to the next tile or
  // segment once the current one is issued) and set up its resources;
  // without one the resources are empty, so the loads read zeros into a
  // stage no one reads.
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
          if (pend0 < 0)
            pend0 = t;
          else
            pend1 = t;
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
    // Slab k0 of the tile: A from column k0 (the range shrinks with it), B
    // from row k0 (the range ends with the slab's last row, so rows past K
    // read zero).
    const int krows = (Kl - k0) < BK ? (Kl - k0) : BK;
    const unsigned long long pa = a_ptr + (unsigned long long)k0 * 2u;
    const unsigned long long pb = b_ptr + (unsigned long long)k0 * (unsigned long long)Nl * 2u;
    rA = rsrc_words_u64(pa, load ? a_rec - (unsigned)k0 * 2u : 0u);
    rB = rsrc_words_u64(pb, load ? (unsigned)(krows * Nl - ln0) * 2u : 0u);
    // Per-lane offsets: the plain ones, except on a K-tail slab or an N-edge
    // tile (and the slab after one), where edge chunks are pushed out of range.
    const bool edge = k0 + BK > Kl || ln0 + BN > Nl;
    if (edge || masked) {
#pragma unroll
      for (int i = 0; i < NA; ++i) ao[i] = (k0 + achk[i] * 8 < Kl) ? aoff[i] : kOob;
#pragma unroll
      for (int i = 0; i < NB; ++i) bo[i] = (ln0 + bchk[i] * 8 < Nl) ? boff[i] : kOob;
      masked = edge;
    }
  };

  // Load d of the prepared slab into stage st.
  auto dma = [&](int st, int d) {
    const unsigned sb = lds0 + (unsigned)(st * S::STAGE);
    if (d < NA)
      load_lds16(rA, sb + (unsigned)((wave * NA + d) * 1024), ao[d]);
    else
      load_lds16(rB, sb + (unsigned)(S::A_BYTES + (wave * NB + d - NA) * 1024), bo[d - NA]);
  };

  f32x4 acc[S::SN][S::SM];
  // MFMA operand fragments, double-buffered by k-step; B^T fragments arrive
  // as two halves (4 k-values each).
  i16x4 bh[2][S::SN][2];
  bf16x8 af[2][S::SM];

  // LDS reads of k-step kk into slot: A block sm (one ds_read_b128), half h
  // of B^T block sn (one transposing read).
  auto read_a = [&](int st, int kk, int slot, int sm) {
    const unsigned char* sbase = smem + st * S::STAGE;
    af[slot][sm] = *reinterpret_cast<const bf16x8*>(sbase + rd_a[kk] + sm * 16 * S::A_ROW);
  };
  auto read_b = [&](int st, int kk, int slot, int sn, int h) {
    const unsigned char* sbase = smem + st * S::STAGE;
    const unsigned char* p = sbase + rd_b[sn] + kk * 32 * S::B_ROW + h * 4 * S::B_ROW;
    bh[slot][sn][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  };

  // MFMA j of k-step `slot`: B^T block j / SM against A block j % SM.  The
  // instruction is written out so that its accumulator operand is an AGPR
  // tuple (left to itself the register allocator moved accumulators between
  // AGPRs and VGPRs around every slab).  The compiler's hazard logic does not
  // see into it, so the code around it keeps the hazards away: a block's
  // accumulator is next read as SrcC NMF MFMAs later, the operand fragments
  // come straight from LDS reads (the compiler waits for those reads before
  // the asm, its inputs), the accumulators are zeroed at the start of a tile
  // with padding after them, and the epilogue reads them only after
  // mfma_results_ready.  tests/test_kernel_hazards.py checks the built code.
  auto mfma = [&](int slot, int j) {
    const int sn = j / S::SM, sm = j % S::SM;
    const bf16x8 b = __builtin_bit_cast(
        bf16x8, __builtin_shufflevector(bh[slot][sn][0], bh[slot][sn][1], 0, 1, 2, 3, 4, 5, 6, 7));
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[sn][sm]) : "v"(b), "v"(af[slot][sm]));
  };

  auto epilogue = [&](int m0, int n0) {
    constexpr unsigned esz = OUT_BF16 ? 2u : 4u;
    const int N = Nc;
    int rows = (Mc - m0) < BM ? (Mc - m0) : BM;
    rows = rows < 0 ? 0 : rows;  // never negative: an empty range drops the stores
    const auto rC = rsrc(static_cast<unsigned char*>(Cc) + ((size_t)m0 * N + n0) * esz,
                         (unsigned)((size_t)rows * N - n0) * esz);
    // lane l holds row l % 16 of a block, columns 4*(l/16) .. +3
    const int r0 = wm * S::TM + l16;
    const int c0 = wn * S::TN + 4 * (lane >> 4);
    const unsigned eb = (unsigned)(r0 * N + c0) * esz;
    const unsigned rstep = 16u * (unsigned)N * esz;
    const int ncols = N - n0;
    if (OUT_BF16) {
      // Two neighbouring blocks at a time: v_permlane16_swap trades the odd
      // 16-lane rows of the first block's packed columns with the even rows
      // of the second's, so lane l holds 8 consecutive columns, (l/32)*8 ..
      // +7, of row l % 16 of block 2*sn2 + (l/16) % 2: one 16-byte store,
      // 64 bytes of each of 16 rows per instruction, the other half of each
      // 128-byte line in the next.  When every row starts on a 128-byte line
      // (N a multiple of 64, C 128-byte aligned) the stores are non-temporal:
      // an XCD's 32 tiles finish together and write 4 MiB of C, as much as
      // its L2, which with the default policy evicted the operand panels the
      // next tiles read (8192^3: +5% under the power limit, +19% at full
      // clock).  With rows off the lines the halves of a line fall to
      // different rows' stores and non-temporal partial lines cost more than
      // they save (3000x7000: -13%), so those keep the default policy.
      const bool nt = N % 64 == 0 && (reinterpret_cast<unsigned long long>(Cc) & 127) == 0;
      const unsigned eb16 = (unsigned)(r0 * N) * 2u;
      const int cl = wn * S::TN + ((lane >> 4) & 1) * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int sm = 0; sm < S::SM; ++sm) {
#pragma unroll
        for (int sn2 = 0; sn2 < S::SN / 2; ++sn2) {
          const f32x4& a = acc[2 * sn2][sm];
          const f32x4& b = acc[2 * sn2 + 1][sm];
          const auto s0 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(a[2], a[3]), pack_bf16x2(b[2], b[3]), false, false);
          const u32x4 v = u32x4{s0[0], s1[0], s0[1], s1[1]};
          const int col = cl + sn2 * 32;
          const unsigned off = col < ncols ? eb16 + sm * rstep + (unsigned)col * 2u : kOob;
          if (nt)
            __builtin_amdgcn_raw_buffer_store_b128(v, rC, off, 0, kAuxNonTemporal);
          else
            __builtin_amdgcn_raw_buffer_store_b128(v, rC, off, 0, 0);
        }
      }
      return;
    }
#pragma unroll
    for (int sm = 0; sm < S::SM; ++sm) {
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn) {
        const int cc = sn * 16;
        const unsigned off = (c0 + cc < ncols) ? eb + sm * rstep + (unsigned)cc * esz : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[sn][sm]), rC, off, 0, 0);
      }
    }
  };

  // Stream-K: the accumulators of a partial segment, fp32, into slot `slot`
  // of this program's workspace ([BM][BN], tile-relative).
  auto store_partial = [&](int slot) {
    float* wsb = P.ws + ((size_t)prog * 2 + slot) * (size_t)(BM * BN);
    const int r0 = wm * S::TM + l16;
    const int c0 = wn * S::TN + 4 * (lane >> 4);
#pragma unroll
    for (int sm = 0; sm < S::SM; ++sm)
#pragma unroll
      for (int sn = 0; sn < S::SN; ++sn) {
        const f32x4& a = acc[sn][sm];
        *reinterpret_cast<f32x4*>(wsb + (r0 + sm * 16) * BN + c0 + sn * 16) = f32x4{a[0], a[1], a[2], a[3]};
      }
  };

  int ct = -1;               // tile on the matrix cores
  int cnsl = nk, cslot = -1;  // its slab count and partial-sum slot (stream-K)
  if (SK) {
    int kb, ke;
    if (cw.next(ct, kb, ke, cslot)) cnsl = ke - kb;
  } else {
    if (tid == 0) s_first[0] = walker.first();
    __syncthreads();
    ct = __builtin_amdgcn_readfirstlane(s_first[0]);
  }
  // Issue order per slab g (stage st = g & 1), fixed by scheduling barriers:
  //   k-step 0: MFMAs; reads of k-step 1; second half of slab g+1's loads
  //   k-steps 1, 2: MFMAs; reads of the next k-step
  //   wait for the wave's loads, barrier: slab g+1 is complete in LDS and
  //   every read of slab g is done, so stage st is free
  //   loader bookkeeping for slab g+2
  //   k-step 3: MFMAs; reads of slab g+1's k-step 0; first half of slab g+2's
  //   loads (into stage st)
  // so the next slab's first fragments and the loads' latency hide behind
  // MFMAs, and each load has at least two k-steps to land.
  constexpr int HALF = NL / 2;
  constexpr int NMH = NMF / 2;  // MFMAs per phase (half a k-step: half the B blocks)
  static_assert(NL % 2 == 0 && HALF <= NMH, "half a slab's loads per phase");
  // Reads of phase ph from stage st_rd, r-th of the phase:
  //   ph 0, 2: the second half of the B^T blocks of k-step ph/2 (slot ph/2),
  //            block SN/2 + r/2, half r&1;
  //   ph 1, 3: k-step 1 (ph 1) or the next slab's k-step 0 (ph 3): B^T block
  //            0, the A blocks, then B^T blocks 1 .. SN/2-1.
  auto phase_read = [&](int ph, int st_rd, int r) {
    if (ph == 0 || ph == 2) {
      const int kk = ph >> 1;
      read_b(st_rd, kk, kk, S::SN / 2 + (r >> 1), r & 1);
    } else {
      const int kk = ph == 1 ? 1 : 0;
      if (r < 2)
        read_b(st_rd, kk, kk, 0, r);
      else if (r < 2 + S::SM)
        read_a(st_rd, kk, kk, r - 2);
      else
        read_b(st_rd, kk, kk, 1 + ((r - 2 - S::SM) >> 1), (r - 2 - S::SM) & 1);
    }
  };
  // Phase ph of a slab: the MFMAs of half (ph & 1) of k-step (ph >> 1), after
  // each its share of the phase's reads and (d0 >= 0) of half a slab's loads.
  auto phase = [&](int ph, int st_rd, int st_dma, int d0) {
    const int kk = ph >> 1, hh = ph & 1;
    const int nrd = (ph == 0 || ph == 2) ? S::SN : S::SM + S::SN;
#pragma unroll
    for (int jl = 0; jl < NMH; ++jl) {
      mfma(kk, hh * NMH + jl);
#pragma unroll
      for (int r = jl * nrd / NMH; r < (jl + 1) * nrd / NMH; ++r) phase_read(ph, st_rd, r);
      if (d0 >= 0) {
#pragma unroll
        for (int d = 0; d < HALF; ++d)
          if (d * NMH / HALF == jl) dma(st_dma, d0 + d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (ct >= 0) {
    if (SK) {
      int v, kb, ke, slot;
      lw.next(v, kb, ke, slot);
      begin_tile(v, kb, ke);
    } else {
      begin_tile(ct, 0, -1);
    }
    prep();  // slab 0
#pragma unroll
    for (int d = 0; d < NL; ++d) dma(0, d);
    wait_vm<0>();
    slab_barrier();
#pragma unroll
    for (int r = 0; r < S::SM + S::SN; ++r) phase_read(3, 0, r);
    prep();  // slab 1: its first half now, the second half in slab 0's phase 0
#pragma unroll
    for (int d = 0; d < HALF; ++d) dma(1, d);
  }

  int g = 0;   // slabs computed so far
  int it = 0;  // tiles finished
  int m0 = 0, n0 = 0;  // origin of tile ct (the loader may already be past it)
  // The matrix cores move on to tile ct: its origin, and (GRP) its problem's
  // output and slab count.
  auto compute_tile = [&]() {
    coords(ct, m0, n0);
    if (GRP) {
      const GemmProblem pr = problem_of(ct);
      Mc = pr.M;
      Nc = pr.N;
      Cc = pr.C;
      cnsl = (pr.K + BK - 1) / BK;
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
        for (int e = 0; e < 4; ++e) acc[sn][sm][e] = 0.0f;
    // wait states between the zeroing writes and the first MFMAs reading them
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    for (int ck = 0; ck < cnsl; ++ck) {
      const int st = g & 1;
      __builtin_amdgcn_sched_barrier(0);
      phase(0, st, st ^ 1, HALF);
      phase(1, st, 0, -1);
      phase(2, st, 0, -1);
      wait_vm<0>();
      slab_barrier();
      prep();  // slab g+2
      __builtin_amdgcn_sched_barrier(0);
      phase(3, st ^ 1, st, 0);
      ++g;
    }
    mfma_results_ready();  // the epilogue reads the accumulators with acc_read
    if (SK && cslot >= 0)
      store_partial(cslot);
    else
      epilogue(m0, n0);
    ++it;
    if (SK) {
      int kb, ke;
      ct = -1;
      if (cw.next(ct, kb, ke, cslot)) cnsl = ke - kb;
    } else {
      ct = pend0;
      pend0 = pend1;
      pend1 = -1;
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

constexpr int kBK = 64;   // slab depth
constexpr int kNST = 2;   // LDS stages

template <int BM, int BN, bool OUT_BF16, bool WITNESS, bool SK = false, bool GRP = false>
hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  using S = Shape<BM, BN, kBK, kNST>;
  auto kern = gemm_bf16_lds_kernel<BM, BN, kBK, kNST, OUT_BF16, WITNESS, SK, GRP>;
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

template <int BM, int BN, bool OUT_BF16, bool GRP = false>
KernelInfo info_one() {
  using S = Shape<BM, BN, kBK, kNST>;
  static const KernelInfo ki = {
      kThreads, S::LDS_BYTES,
      occupancy_of(reinterpret_cast<const void*>(
                       gemm_bf16_lds_kernel<BM, BN, kBK, kNST, OUT_BF16, false, false, GRP>),
                   kThreads, S::LDS_BYTES)};
  return ki;
}

// Stream-K fix-up.  Each tile of the stream-K part is cut into
// kFixBands bands of rows; block (v - dp) * kFixBands + band sums its band of
// tile v from the partial-sum slots of the programs whose runs share the
// tile, in slab order, and stores it (rows past M and columns past N
// dropped).  Tiles one program computed whole were stored by that program.
// Bands give the memory-bound pass many more blocks than tiles; each thread
// keeps kFixVec independent 16-byte loads in flight per contributor.
constexpr int kFixBands = 8;
constexpr int kFixThreads = 256;

template <int BM, int BN, bool OUT_BF16>
__global__ void __launch_bounds__(kFixThreads) sk_fixup_kernel(SkFixParams F) {
  constexpr int kBandElems = BM * BN / kFixBands;
  constexpr int kFixVec = kBandElems / (kFixThreads * 4);
  static_assert(kFixVec >= 1 && kBandElems % (kFixThreads * 4) == 0, "band shape");
  const int v = F.dp + (int)(blockIdx.x / kFixBands);
  const int band = (int)(blockIdx.x % kFixBands);
  if (v >= F.T) return;
  const long long j0 = (long long)(v - F.dp) * F.nk;
  const int q0 = pgs::sk_owner(j0, F.W, F.G), q1 = pgs::sk_owner(j0 + F.nk - 1, F.W, F.G);
  if (q0 == q1) return;
  int pm, pn;
  pgs::decode(pgs::kStreamK, v, F.num_pid_m, F.num_pid_n, F.gs, pm, pn);
  const int m0 = pm * BM, n0 = pn * BN;
  const int e0 = band * kBandElems + threadIdx.x * 4;
  f32x4 sum[kFixVec];
#pragma unroll
  for (int i = 0; i < kFixVec; ++i) sum[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int q = q0; q <= q1; ++q) {
    if (pgs::sk_run_begin(q, F.W, F.G) == pgs::sk_run_begin(q + 1, F.W, F.G)) continue;
    const int slot = pgs::sk_slot(q, v, F.dp, F.nk, F.W, F.G);
    const f32x4* src = reinterpret_cast<const f32x4*>(F.ws + ((size_t)q * 2 + slot) * (size_t)(BM * BN) + e0);
    f32x4 x[kFixVec];
#pragma unroll
    for (int i = 0; i < kFixVec; ++i) x[i] = __builtin_nontemporal_load(src + i * kFixThreads);
#pragma unroll
    for (int i = 0; i < kFixVec; ++i) sum[i] += x[i];
  }
#pragma unroll
  for (int i = 0; i < kFixVec; ++i) {
    const int e = e0 + i * kFixThreads * 4;
    const int r = m0 + e / BN, c = n0 + e % BN;
    if (r >= F.M || c >= F.N) continue;  // N % 8 == 0: the 4 columns are all in or all out
    if (OUT_BF16) {
      unsigned short* C = static_cast<unsigned short*>(F.C);
      *reinterpret_cast<u32x2*>(C + (size_t)r * F.N + c) =
          u32x2{pack_bf16x2(sum[i][0], sum[i][1]), pack_bf16x2(sum[i][2], sum[i][3])};
    } else {
      float* C = static_cast<float*>(F.C);
      *reinterpret_cast<f32x4*>(C + (size_t)r * F.N + c) = sum[i];
    }
  }
}

template <int BM, int BN>
hipError_t launch_tile(const GemmParams& p, bool out_bf16, bool witness, hipStream_t stream) {
  if (out_bf16)
    return witness ? launch_one<BM, BN, true, true>(p, stream) : launch_one<BM, BN, true, false>(p, stream);
  return witness ? launch_one<BM, BN, false, true>(p, stream) : launch_one<BM, BN, false, false>(p, stream);
}

}  // namespace

// The direct-to-LDS path: needs 16-byte aligned rows of A, B and C, and the
// 32-bit buffer offsets of one tile panel / slab to stay in range.
bool gemm_bf16_lds_eligible(int bm, int bn, int bk, long long N, long long K) {
  if (bk != 64) return false;
  if (!((bm == 256 && bn == 256) || (bm == 128 && bn == 128))) return false;
  if (K % 8 != 0 || N % 8 != 0) return false;
  return (long long)bm * K * 2 < (1LL << 31) && 64LL * N * 2 < (1LL << 31) &&
         (long long)bm * N * 4 < (1LL << 31);
}

KernelInfo info_gemm_bf16_lds(int bm, int bn, bool out_bf16) {
  if (bm == 256 && bn == 256) return out_bf16 ? info_one<256, 256, true>() : info_one<256, 256, false>();
  if (bm == 128 && bn == 128) return out_bf16 ? info_one<128, 128, true>() : info_one<128, 128, false>();
  return KernelInfo{0, 0, 0};
}

hipError_t launch_gemm_bf16_lds_sk(const GemmParams& p, int bm, int bn, bool out_bf16,
                                   hipStream_t stream) {
  if (bm == 256 && bn == 256)
    return out_bf16 ? launch_one<256, 256, true, false, true>(p, stream)
                    : launch_one<256, 256, false, false, true>(p, stream);
  if (bm == 128 && bn == 128)
    return out_bf16 ? launch_one<128, 128, true, false, true>(p, stream)
                    : launch_one<128, 128, false, false, true>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_sk_fixup(const SkFixParams& f, int bm, int bn, bool out_bf16, hipStream_t stream) {
  if (f.T - f.dp <= 0) return hipSuccess;
  const dim3 blocks((unsigned)(f.T - f.dp) * kFixBands), threads(kFixThreads);
  if (bm == 256 && bn == 256) {
    if (out_bf16)
      hipLaunchKernelGGL((sk_fixup_kernel<256, 256, true>), blocks, threads, 0, stream, f);
    else
      hipLaunchKernelGGL((sk_fixup_kernel<256, 256, false>), blocks, threads, 0, stream, f);
  } else if (bm == 128 && bn == 128) {
    if (out_bf16)
      hipLaunchKernelGGL((sk_fixup_kernel<128, 128, true>), blocks, threads, 0, stream, f);
    else
      hipLaunchKernelGGL((sk_fixup_kernel<128, 128, false>), blocks, threads, 0, stream, f);
  } else if (bm == 128 && bn == 256 && out_bf16) {  // the fp8 kernel's 128x256 tile
    hipLaunchKernelGGL((sk_fixup_kernel<128, 256, true>), blocks, threads, 0, stream, f);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_lds_grouped(const GemmParams& p, int bm, int bn, bool out_bf16, bool witness,
                                        hipStream_t stream) {
  if (p.ngemm < 1 || p.ngemm > kMaxGemmProblems) return hipErrorInvalidValue;
  if (bm == 256 && bn == 256) {
    if (out_bf16)
      return witness ? launch_one<256, 256, true, true, false, true>(p, stream)
                     : launch_one<256, 256, true, false, false, true>(p, stream);
    return witness ? launch_one<256, 256, false, true, false, true>(p, stream)
                   : launch_one<256, 256, false, false, false, true>(p, stream);
  }
  if (bm == 128 && bn == 128) {
    if (out_bf16)
      return witness ? launch_one<128, 128, true, true, false, true>(p, stream)
                     : launch_one<128, 128, true, false, false, true>(p, stream);
    return witness ? launch_one<128, 128, false, true, false, true>(p, stream)
                   : launch_one<128, 128, false, false, false, true>(p, stream);
  }
  return hipErrorInvalidValue;
}

KernelInfo info_gemm_bf16_lds_grouped(int bm, int bn, bool out_bf16) {
  if (bm == 256 && bn == 256)
    return out_bf16 ? info_one<256, 256, true, true>() : info_one<256, 256, false, true>();
  if (bm == 128 && bn == 128)
    return out_bf16 ? info_one<128, 128, true, true>() : info_one<128, 128, false, true>();
  return KernelInfo{0, 0, 0};
}

hipError_t launch_gemm_bf16_lds(const GemmParams& p, int bm, int bn, bool out_bf16, bool witness,
                                hipStream_t stream) {
  if (bm == 256 && bn == 256) return launch_tile<256, 256>(p, out_bf16, witness, stream);
  if (bm == 128 && bn == 128) return launch_tile<128, 128>(p, out_bf16, witness, stream);
  return hipErrorInvalidValue;
}

}  // namespace pgk
