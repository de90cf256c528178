// Persistent bf16 GEMM for gfx950 with two wave groups in ping-pong:
// C[M][N] = A[M][K] . B[K][N], fp32 accumulate, 256x256x64 tiles.
//
// The persistent tile loop and the schedulers are those of the other bf16
// kernels ("Work Stealing Scheduler Kernel", tritonBLAS PR #65;
// "Implement persistent kernels", Helion PR #238).  What this kernel adds is
// the pipeline of "[Feature] Introduce tile scheduler" (TileLang PR #2441,
// MXFP8 example): there, warps take roles (load, MMA, epilogue), each role
// walks the tile sequence with its own scheduler instance, and the epilogue
// drains finished accumulators while the MMA role already works on the next
// tile.  A gfx950 SIMD has no separate tensor memory to hand accumulators
// over and cannot hold a fifth register-heavy wave, so the roles are
// re-cut for CDNA4:
//  * Eight waves, two per SIMD (waves w and w+4 share SIMD w mod 4).  Group 0
//    (waves 0-3) computes columns 0..127 of the tile and group 1 (waves
//    4-7) columns 128..255; each wave owns a 128x64 sub-tile (8 blocks of
//    v_mfma_f32_32x32x16_bf16, 128 accumulator registers, placed by the
//    compiler: with 256 registers per wave the accumulators and the
//    fragments fit in VGPRs, and MFMAs read and write VGPRs as fast).
//  * The groups alternate: while one group's waves issue MFMAs (two k-steps,
//    16 MFMAs per wave, at raised wave priority), the other group's waves read
//    their next fragments from LDS, issue global loads or drain a finished
//    tile; a workgroup barrier separates the phases, and group 1 runs one
//    phase behind group 0, so every SIMD always has one wave with matrix work
//    and one with memory work.  LDS waits and a group's epilogue sit under
//    the other group's MFMAs.
//  * Group 0 is the loader: it issues every global -> LDS load (16 KiB per
//    wave per slab), three phases before the slab is read, always ahead of
//    its own C stores, so its load waits never wait for stores it issued
//    later (vector memory operations retire in issue order).  Group 1 issues
//    no loads, so its C stores never stall a load wait at all.
//  * The tile sequence is claimed by thread 0 (the loader side, one slab
//    ahead of the loads) and published in a small LDS ring; both groups'
//    compute sides read the ids from the ring, so each group walks the same
//    sequence with its own cursor.
//  * LDS: two stages of one 64-deep slab (A [256][64] + B [64][256] bf16,
//    128 KiB), the layout and swizzles of the four-wave kernel; B^T
//    fragments by ds_read_b64_tr_b16, A fragments by ds_read_b128.
//  * Masked edges as in the other kernels: rows past M / K read zero through
//    the buffer range check, the K tail and columns past N are masked per
//    lane, C stores outside the matrix are dropped; no index wrapping.
#include "common.hpp"
#include "gemm_device.hpp"

namespace pgk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

namespace pp {
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TM = 128, TN = 64;              // one wave's sub-tile
constexpr int SM = TM / 32, SN = TN / 32;     // 4 x 2 MFMA blocks
constexpr int NMF = SM * SN;                  // MFMAs per wave per k-step
constexpr int NRD = 2 * SN + SM;              // LDS reads per wave per k-step
constexpr int A_ROW = BK * 2;                 // bytes per LDS row of A
constexpr int A_BYTES = BM * A_ROW;           // one stage of A (32 KiB)
constexpr int B_ROW = BN * 2;                 // bytes per LDS row of B
constexpr int B_BYTES = BK * B_ROW;           // one stage of B (32 KiB)
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int RING = 8;                       // tile-id ring entries
constexpr int LDS_BYTES = 2 * STAGE + RING * 4;
constexpr int LOADERS = 4;                    // group 0 issues every load
constexpr int NA = A_BYTES / 1024 / LOADERS;  // 1 KiB loads per loader wave per slab
constexpr int NB = B_BYTES / 1024 / LOADERS;
constexpr int NL = NA + NB;
constexpr int A_RPI = 1024 / A_ROW, A_CPR = A_ROW / 16;
constexpr int B_RPI = 1024 / B_ROW, B_CPR = B_ROW / 16;
static_assert(NA * LOADERS * 1024 == A_BYTES && NB * LOADERS * 1024 == B_BYTES, "slab splits into loads");
static_assert(NL <= 16, "loads of one slab fit the vmcnt wait below");
}  // namespace pp

__device__ __forceinline__ void phase_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

template <bool OUT_BF16, bool WITNESS>
__global__ void __launch_bounds__(pp::kThreads) gemm_bf16_pp_kernel(GemmParams P) {
  using namespace pp;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  int* s_ring = reinterpret_cast<int*>(smem + 2 * STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;        // 0: loader + left half, 1: right half
  const int q = wave & 3;
  const int wm = q >> 1;            // rows wm*128 ..
  const int wn = grp * 2 + (q & 1); // columns wn*64 ..
  const int prog = pgs::program_of(blockIdx.x, P.s.G, P.s.X, P.s.xcd_major);
  const int M = P.M, N = P.N, K = P.K;
  const unsigned short* Ag = static_cast<const unsigned short*>(P.A);
  const unsigned short* Bg = static_cast<const unsigned short*>(P.B);

  Walker walker(P.s, prog);
  if (WITNESS) walker.claim_row = P.w.claims + (size_t)prog * kMaxStealCounters;
  long long t_start = 0, c_start = 0;
  if (WITNESS && tid == 0) {
    t_start = wall_ticks();
    c_start = shader_cycles();
  }

  // ---- loader lane offsets (group 0): load q*NA + i of A covers rows
  // A_RPI*(q*NA + i) ..; the lane's LDS chunk p % CPR holds global chunk
  // bf16_swz_a(row, p % CPR) (an involution), likewise for B.
  auto a_chk = [&](int i) {
    const int row = (q * NA + i) * A_RPI + lane / A_CPR;
    return bf16_swz_a<BK>(row, lane % A_CPR);
  };
  auto b_chk = [&](int i) {
    const int row = (q * NB + i) * B_RPI + lane / B_CPR;
    return bf16_swz_b(row, lane % B_CPR);
  };
  unsigned aoff[NA], boff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = (q * NA + i) * A_RPI + lane / A_CPR;
    aoff[i] = (unsigned)row * (unsigned)K * 2u + (unsigned)a_chk(i) * 16u;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = (q * NB + i) * B_RPI + lane / B_CPR;
    boff[i] = (unsigned)row * (unsigned)N * 2u + (unsigned)b_chk(i) * 16u;
  }
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  // ---- LDS read offsets of the wave's fragments ----
  const int l32 = lane & 31;
  unsigned rd_a[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int row = wm * TM + l32;
    rd_a[kk] = (unsigned)(row * A_ROW + bf16_swz_a<BK>(row, kk * 2 + (lane >> 5)) * 16);
  }
  unsigned rd_b[SN];
  {
    const int g = lane >> 4, i16 = lane & 15, a = i16 & 3, e = i16 >> 2;
    const int krow = (g >> 1) * 8 + e;  // + kk*16 + h*4 (multiples of 4: swizzle unchanged)
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
      const int n = wn * TN + sn * 32 + (g & 1) * 16 + 4 * a;
      const int c = bf16_swz_b(krow, n >> 3);
      rd_b[sn] = (unsigned)(A_BYTES + krow * B_ROW + c * 16 + 8 * (a & 1));
    }
  }

  const int nk = (K + BK - 1) / BK;

  // ---- loader state (group 0) ----
  int lt = -1, lk = 0;      // loader tile and its next slab
  int lo = 0;               // ordinal of the loader tile in the program's sequence
  int lm0 = 0, ln0 = 0;
  unsigned long long a_ptr = 0, b_ptr = 0;
  unsigned a_rec = 0;
  rsrc_words_t rA, rB;
  bool load = false;
  bool edge = false;        // K-tail slab or N-edge tile: chunks past K / N masked per lane
  int kleft = 0, nleft = 0; // K - k0 and N - n0 of the prepared slab

  auto begin_tile = [&](int t) {
    lt = t;
    lk = 0;
    int pm, pn;
    walker.tile_coords(t, pm, pn);
    lm0 = pm * BM;
    ln0 = pn * BN;
    int rows = (M - lm0) < BM ? (M - lm0) : BM;
    rows = rows < 0 ? 0 : rows;
    a_ptr = reinterpret_cast<unsigned long long>(Ag + (size_t)lm0 * K);
    a_rec = (unsigned)(rows * K) * 2u;
    b_ptr = reinterpret_cast<unsigned long long>(Bg + ln0);
  };

  // Set up the loader's next slab, moving to the next tile of the sequence
  // (published in the ring one slab earlier) once the current one is issued.
  // The next tile is claimed when the last slab of the current one is set up.
  auto prep = [&]() {
    lt = __builtin_amdgcn_readfirstlane(lt);
    lk = __builtin_amdgcn_readfirstlane(lk);
    lo = __builtin_amdgcn_readfirstlane(lo);
    if (lt >= 0 && lk == nk) {
      const int t = __builtin_amdgcn_readfirstlane(s_ring[(lo + 1) & (RING - 1)]);
      ++lo;
      lt = -1;
      if (t >= 0) begin_tile(t);
    }
    const int k0 = lk * BK;
    load = lt >= 0;
    if (load) {
      ++lk;
      if (lk == nk && wave == 0) {  // the whole wave claims, so the walk stays uniform
        const int t = walker.next_wave(lt);
        if (lane == 0) s_ring[(lo + 1) & (RING - 1)] = t;
      }
    }
    const int krows = (K - k0) < BK ? (K - k0) : BK;
    rA = rsrc_words_u64(a_ptr + (unsigned long long)k0 * 2u, load ? a_rec - (unsigned)k0 * 2u : 0u);
    rB = rsrc_words_u64(b_ptr + (unsigned long long)k0 * (unsigned long long)N * 2u,
                        load ? (unsigned)(krows * N - ln0) * 2u : 0u);
    edge = k0 + BK > K || ln0 + BN > N;
    kleft = K - k0;
    nleft = N - ln0;
  };

  // All of the prepared slab's loads of this wave into stage st.
  auto dma_all = [&](int st) {
    if (!load) return;
    const unsigned sb = lds0 + (unsigned)(st * STAGE);
    if (edge) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        load_lds16(rA, sb + (unsigned)((q * NA + i) * 1024), a_chk(i) * 8 < kleft ? aoff[i] : kOob);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        load_lds16(rB, sb + (unsigned)(A_BYTES + (q * NB + i) * 1024), b_chk(i) * 8 < nleft ? boff[i] : kOob);
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) load_lds16(rA, sb + (unsigned)((q * NA + i) * 1024), aoff[i]);
#pragma unroll
      for (int i = 0; i < NB; ++i) load_lds16(rB, sb + (unsigned)(A_BYTES + (q * NB + i) * 1024), boff[i]);
    }
  };

  f32x16 acc[SN][SM];
  // fragments of the two k-steps of the next compute phase
  i16x4 bh[2][SN][2];
  bf16x8 af[2][SM];

  // Fragment reads of k-steps 2h and 2h+1 of stage st: per k-step B^T block
  // halves first, then the A blocks.
  auto read_half = [&](int st, int h) {
    const unsigned char* sbase = smem + st * STAGE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = 2 * h + s;
#pragma unroll
      for (int sn = 0; sn < SN; ++sn)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const unsigned char* p = sbase + rd_b[sn] + kk * 16 * B_ROW + hh * 4 * B_ROW;
          bh[s][sn][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
        }
#pragma unroll
      for (int sm = 0; sm < SM; ++sm)
        af[s][sm] = *reinterpret_cast<const bf16x8*>(sbase + rd_a[kk] + sm * 32 * A_ROW);
    }
  };

  // 16 MFMAs: the two k-steps whose fragments were read in the last memory phase.
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int sn = 0; sn < SN; ++sn)
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(bh[s][sn][0], bh[s][sn][1], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, af[s][sm], acc[sn][sm], 0, 0, 0);
        }
    __builtin_amdgcn_s_setprio(0);
  };

  auto zero_acc = [&]() {
#pragma unroll
    for (int sn = 0; sn < SN; ++sn)
#pragma unroll
      for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[sn][sm][e] = 0.0f;
  };

  // Store the wave's 128x64 sub-tile of the tile at (m0, n0).
  auto epilogue = [&](int m0, int n0) {
    constexpr unsigned esz = OUT_BF16 ? 2u : 4u;
    int rows = (M - m0) < BM ? (M - m0) : BM;
    rows = rows < 0 ? 0 : rows;
    const auto rC = rsrc(static_cast<unsigned char*>(P.C) + ((size_t)m0 * N + n0) * esz,
                         (unsigned)((size_t)rows * N - n0) * esz);
    const int r0 = wm * TM + l32;
    const unsigned rstep = 32u * (unsigned)N * esz;
    const int ncols = N - n0;
    if (OUT_BF16) {
      const int hi = lane >> 5;
      const unsigned eb2 = (unsigned)(r0 * N) * 2u;
#pragma unroll
      for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn)
          store_block_bf16<false>(acc[sn][sm], rC, eb2 + sm * rstep, wn * TN + sn * 32, ncols, hi);
    } else {
      const int c0 = wn * TN + 4 * (lane >> 5);
      const unsigned eb = (unsigned)(r0 * N + c0) * esz;
#pragma unroll
      for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int cc = sn * 32 + 8 * g;
            const unsigned off = (c0 + cc < ncols) ? eb + sm * rstep + (unsigned)cc * esz : kOob;
            const f32x16& a = acc[sn][sm];
            const f32x4 v = f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rC, off, 0, 0);
          }
    }
  };
  // C stores one epilogue issues per wave (vmcnt counts them)
  constexpr int NST = OUT_BF16 ? SM * SN * 2 : SM * SN * 4;
  static_assert(NST <= 63, "stores of one epilogue fit the vmcnt field");

  // ---- prologue: slabs 0 and 1 in flight, slab 0 complete ----
  if (wave == 0) {
    const int t = walker.first_wave();
    if (lane == 0) s_ring[0] = t;
  }
  __syncthreads();
  int ct = __builtin_amdgcn_readfirstlane(s_ring[0]);
  int it = 0;  // tiles finished by this program (witness)
  if (ct >= 0) {
    int co = 0;  // ordinal of tile ct in the program's sequence
    int ck = 0;  // slab of tile ct on the matrix cores
    int g = 0;   // slabs so far (stage g & 1)
    int pm, pn;
    walker.tile_coords(ct, pm, pn);
    int m0 = pm * BM, n0 = pn * BN;
    if (grp == 0) {
      begin_tile(ct);
      prep();  // slab 0 (claims the next tile if the first has one slab)
      dma_all(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    phase_barrier();  // the claim is visible to the other loader waves
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) {
      prep();  // slab 1
      dma_all(1);
      // this wave's loads of slab 0 (slab 1's, if any, may stay in flight)
      if (load)
        wait_vm<NL>();
      else
        wait_vm<0>();
    }
    zero_acc();
    bool stored = false;  // an epilogue's stores were issued after the loads of the next slab
    __builtin_amdgcn_sched_barrier(0);
    phase_barrier();  // slab 0 complete in LDS
    // Group 1 runs one phase behind group 0: it passes one barrier more here
    // and group 0 one more after the loop, so the k-th barrier of group 1's
    // loop meets the (k+1)-th of group 0's, and each SIMD's two waves
    // alternate between the memory and the compute phases below.
    if (grp == 1) phase_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // One iteration per slab g of tile ct, in four phases, each closed by a
    // barrier: fragments of k-steps 0-1, their MFMAs, fragments of k-steps
    // 2-3, their MFMAs.  The stage of slab g is read in the two memory phases
    // of both groups and is free once group 1's second one has passed, which
    // is group 0's fourth barrier; group 0 then loads slab g+2 into it and
    // waits for those loads at its fourth barrier one slab later, three
    // phases on.
    for (;;) {
      const int st = g & 1;
      const bool last = ck == nk - 1;
      if (ck == 0 && tid == 0) {
        if (WITNESS) {
          atomicAdd(P.w.visits + ct, 1);
          P.w.owner[ct] = prog;
          P.w.order[ct] = it;
        }
        if (is_straggler(P.s, prog)) spin_ns(P.s.straggler_ns, P.s.wall_khz);
      }
      read_half(st, 0);
      __builtin_amdgcn_sched_barrier(0);
      slab_barrier();
      __builtin_amdgcn_sched_barrier(0);
      compute();
      __builtin_amdgcn_sched_barrier(0);
      phase_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_half(st, 1);
      __builtin_amdgcn_sched_barrier(0);
      slab_barrier();
      __builtin_amdgcn_sched_barrier(0);
      compute();
      __builtin_amdgcn_sched_barrier(0);
      if (grp == 0) {
        // the loads of slab g+1 (issued a slab ago, before any stores issued
        // with them) are done; the barrier publishes the slab
        if (stored)
          wait_vm<NST>();
        else
          wait_vm<0>();
      }
      phase_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (grp == 0) {
        prep();  // slab g+2, into the stage slab g leaves
        dma_all(st);
      }
      stored = false;
      ++g;
      if (!last) {
        ++ck;
        continue;
      }
      // tile ct is done: drain it (under the other group's MFMAs) and move on
      epilogue(m0, n0);
      stored = true;
      ++it;
      const int nt = __builtin_amdgcn_readfirstlane(s_ring[(co + 1) & (RING - 1)]);
      if (nt < 0) break;
      zero_acc();
      ct = nt;
      ++co;
      ck = 0;
      walker.tile_coords(ct, pm, pn);
      m0 = pm * BM;
      n0 = pn * BN;
    }
    if (grp == 0) phase_barrier();
  }

  if (WITNESS && tid == 0) {
    P.w.t_start[prog] = t_start;
    P.w.t_end[prog] = wall_ticks();
    P.w.cycles[prog] = shader_cycles() - c_start;
    P.w.hw_id[prog] = hw_placement();
    P.w.n_tiles[prog] = it;
  }
}

template <bool OUT_BF16, bool WITNESS>
hipError_t launch_pp(const GemmParams& p, hipStream_t stream) {
  auto kern = gemm_bf16_pp_kernel<OUT_BF16, WITNESS>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, pp::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.s.G), dim3(pp::kThreads), pp::LDS_BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace

// The ping-pong kernel takes 256x256x64 tiles on the direct-to-LDS terms
// (16-byte aligned rows, K and N multiples of 8, one tile's panels within
// 32-bit byte offsets), one problem, data-parallel and work-stealing
// schedulers.
bool gemm_bf16_pp_eligible(int bm, int bn, int bk, long long N, long long K) {
  return bm == 256 && bn == 256 && gemm_bf16_lds_eligible(bm, bn, bk, N, K);
}

KernelInfo info_gemm_bf16_pp(bool out_bf16) {
  static const KernelInfo kb = {
      pp::kThreads, pp::LDS_BYTES,
      occupancy_of(reinterpret_cast<const void*>(gemm_bf16_pp_kernel<true, false>), pp::kThreads,
                   pp::LDS_BYTES)};
  static const KernelInfo kf = {
      pp::kThreads, pp::LDS_BYTES,
      occupancy_of(reinterpret_cast<const void*>(gemm_bf16_pp_kernel<false, false>), pp::kThreads,
                   pp::LDS_BYTES)};
  return out_bf16 ? kb : kf;
}

hipError_t launch_gemm_bf16_pp(const GemmParams& p, bool out_bf16, bool witness, hipStream_t stream) {
  if (out_bf16) return witness ? launch_pp<true, true>(p, stream) : launch_pp<true, false>(p, stream);
  return witness ? launch_pp<false, true>(p, stream) : launch_pp<false, false>(p, stream);
}

}  // namespace pgk
