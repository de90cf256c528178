// Device helpers shared by the direct-to-LDS MFMA GEMM kernels (gfx950):
// buffer resources, global -> LDS loads, waits and barriers, accumulator
// reads and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>

namespace pgk {

// A buffer offset past every range: the load returns zeros, a store is dropped.
constexpr unsigned kOob = 0x80000000u;
// Buffer resource word 3 for raw (unformatted, unswizzled) byte buffers.
constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over [base, base + bytes); base and bytes are uniform
// across the wave and readfirstlane says so, so the resource lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  void* ub = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           kRsrcWord3);
}

typedef unsigned rsrc_words_t __attribute__((ext_vector_type(4)));

// The same resource as four SGPR words, for the hand-issued loads below.
__device__ __forceinline__ rsrc_words_t rsrc_words(const void* base, unsigned bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  return rsrc_words_t{(unsigned)__builtin_amdgcn_readfirstlane((unsigned)b),
                      (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) & 0xffffu,
                      (unsigned)__builtin_amdgcn_readfirstlane(bytes), (unsigned)kRsrcWord3};
}

__device__ __forceinline__ rsrc_words_t rsrc_words_u64(unsigned long long base, unsigned bytes) {
  return rsrc_words_t{(unsigned)__builtin_amdgcn_readfirstlane((unsigned)base),
                      (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(base >> 32)) & 0xffffu,
                      (unsigned)__builtin_amdgcn_readfirstlane(bytes), (unsigned)kRsrcWord3};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(unsigned long)((const __attribute__((address_space(3))) void*)p);
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from byte offset voff of
// the buffer into LDS at lds_dst + 16 * lane (lds_dst uniform).  Issued by
// hand: the compiler would treat the intrinsic form as an LDS store of
// unknown extent and wait for every such load still in flight (vmcnt(0))
// before each later LDS read, which serialises the slab pipeline.  The
// kernels track completion themselves: s_waitcnt vmcnt on the issuing wave,
// then a workgroup barrier, before any wave reads the slab.
//
// Both asm statements below write M0 and list it as clobbered, so the
// compiler does not keep a value of its own in M0 across them.  M0 is a
// reserved register to the AMDGPU backend, which warns about the clobber;
// the warning is silenced for these two statements only.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(rsrc_words_t r, unsigned lds_address, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_address), "v"(voff), "s"(r) : "memory", "m0");
}

// buffer_load_ubyte ... lds: one byte per lane from byte offset voff,
// written zero-extended to the LDS dword at M0 + 4 * lane (bytes past the
// resource's range read as zero).
__device__ __forceinline__ void load_lds_u8(rsrc_words_t r, unsigned lds_address, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ubyte %1, %2, 0 offen lds"
               :: "s"(lds_address), "v"(voff), "s"(r) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void load_lds16(rsrc_words_t r, unsigned char* lds_dst, unsigned voff) {
  load_lds16(r, __builtin_amdgcn_readfirstlane(lds_addr(lds_dst)), voff);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// half waits for every outstanding global access): the caller has already
// waited (vmcnt) for the LDS loads the other waves will read; this waits for
// the wave's own LDS reads and writes, then meets the other waves.
__device__ __forceinline__ void slab_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copy one accumulator out of its AGPR.  Spelling the read out keeps the
// register allocator from moving all accumulators to VGPRs (the conversion
// to bf16 is a VALU instruction and cannot read AGPRs).
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// Wait for the results of the MFMAs issued so far before acc_read touches
// them.  The hazard logic of the compiler does not look into the inline asm
// of acc_read, so it neither keeps those reads after the MFMAs that write the
// accumulators nor pads them with the wait states an MFMA result needs
// (16-pass XDL write, then VALU read: 18).  Call it after the tile's last
// MFMA: 24 wait states cover that MFMA, and every earlier one finished
// before it.  The sched_barriers keep MFMAs and reads on their own side.
__device__ __forceinline__ void mfma_results_ready() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Two floats rounded to bf16 (nearest even) and packed, the first in the
// low half.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// LDS layout of the bf16 kernels' operand slabs.
// LDS banks: 64 x 4 bytes.  A ds_read_b128 is served 16 lanes at a time and
// a ds_read_b64 (also the transposing form) 32 lanes at a time, so a read is
// conflict-free when those lanes hit distinct 16- (8-) byte slots of a
// 256-byte window.
//
// Physical chunk of logical chunk c in row `row` of A: the MFMA operand read
// touches 16 consecutive rows at one logical chunk; the XOR spreads them
// over the 16 slots (128-byte rows: 2 rows per window x 8 chunks; 64-byte
// rows: 4 rows x 4 chunks).
template <int BK>
__device__ __forceinline__ int bf16_swz_a(int row, int c) {
  return BK == 64 ? (c ^ ((row >> 1) & 7)) : (c ^ ((row >> 2) & 3));
}

// Physical chunk of logical chunk c in row k of B: a transposing read of 32
// lanes touches 4 consecutive rows x 4 consecutive chunks; XOR-ing chunk
// bits 2-3 with the row moves the 4 rows to different quarter windows.
__device__ __forceinline__ int bf16_swz_b(int k, int c) { return c ^ (4 * (k & 3)); }

// Store one 32x32 block of fp32 accumulators as bf16.  Layout of
// v_mfma_f32_32x32 with B^T as the first operand: lane l holds row l % 32,
// columns 8g + 4*(l/32) .. +3 in registers 4g .. 4g+3 (g = 0..3).  Swapping
// the g = 2q+1 half of the low 32 lanes with the g = 2q half of the high 32
// (v_permlane32_swap: r0 = [a.lo | b.lo], r1 = [a.hi | b.hi]) leaves each
// lane 8 consecutive columns, the low lane those of g = 2q and the high lane
// those of g = 2q+1, stored as one 16-byte chunk.  row_off: byte offset of
// the lane's row at column 0 of the block's tile; col0: the block's first
// column; chunks at or past ncols are dropped (ncols a multiple of 8).
// AGPR_READS: read each accumulator with an explicit v_accvgpr_read (for
// kernels whose accumulators must stay in AGPRs); otherwise the compiler
// places them.
template <bool AGPR_READS = true, typename Acc>
__device__ __forceinline__ void store_block_bf16(const Acc& a, __amdgpu_buffer_rsrc_t rC,
                                                 unsigned row_off, int col0, int ncols, int hi) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  auto rd = [&](int i) { return AGPR_READS ? acc_read(a[i]) : a[i]; };
  unsigned pk[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    pk[g][0] = pack_bf16x2(rd(4 * g), rd(4 * g + 1));
    pk[g][1] = pack_bf16x2(rd(4 * g + 2), rd(4 * g + 3));
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * q][0], pk[2 * q + 1][0], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * q][1], pk[2 * q + 1][1], false, false);
    const u32x4_t v = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
    const int col = col0 + 8 * (2 * q + hi);
    const unsigned off = col < ncols ? row_off + (unsigned)col * 2u : kOob;
    __builtin_amdgcn_raw_buffer_store_b128(v, rC, off, 0, 0);
  }
}

}  // namespace pgk
