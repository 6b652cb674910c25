// Shared device helpers for the gfx950 attention kernels: vector types, bf16 MFMA,
// LDS reads (plain and transposing), packing. CDNA4 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies A row (l % 32), k = 8*(l/32) .. +7, and B column (l % 32), same k.
// Lane l receives D column (l % 32), rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 contiguous bytes from LDS.
__device__ __forceinline__ bf16x8 lds_b128(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, lane i
// points at 4 consecutive bf16 of a row-major tile; lane j gets back element e
// = the (j%4)-th element of lane (4e + j/4)'s four. Point lane i at
// tile[r0 + i/4][c0 + 4*(i%4)] and lane j receives tile[r0 .. r0+3][c0 + j]:
// one column, four consecutive rows.
__device__ __forceinline__ i16x4 lds_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_char*)p));
}

__device__ __forceinline__ bf16x8 cat(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Eight fp32 -> eight bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  f32x8 x = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(x, bf16x8);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a0, float a1, float a2, float a3) {
  f32x4 x = {a0, a1, a2, a3};
  return __builtin_convertvector(x, bf16x4);
}

// Exchange with the lane 32 away (the other half of the wave). v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with both holding x, the lower lanes of the second result and the
// upper lanes of the first hold the other half's values. Two VALU operations,
// no trip through LDS as with a general lane shuffle.
__device__ __forceinline__ float swap_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (__lane_id() & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

}  // namespace fa

namespace fa {

// ------------------------------------------------------------------------------------------------
// Swizzled LDS tiles filled by direct global->LDS loads.
//
// A tile has rows of C 16-byte chunks (C = 8 or 16), stored without padding;
// chunk c of row r sits at chunk position c ^ swz<C>(r). The permutation makes
// both access patterns of the kernels free of LDS bank conflicts: 16-byte reads
// of 16 consecutive rows at one chunk (MFMA operands read along the row) and
// transposing 8-byte reads of 4 consecutive rows x 4 consecutive chunks.
template <int C>
__device__ __forceinline__ int swz(int r);
template <>
__device__ __forceinline__ int swz<16>(int r) {
  return ((r & 3) << 2) | ((r >> 2) & 3);
}
template <>
__device__ __forceinline__ int swz<8>(int r) {
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of (row r, column col) in a swizzled tile with rows of C chunks.
template <int C>
__device__ __forceinline__ int toff(int r, int col) {
  return r * (8 * C) + ((((col >> 3) ^ swz<C>(r)) & (C - 1)) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane
// l writes LDS bytes [lds + 16 l, lds + 16 l + 16). Issued through asm so that
// the compiler does not treat it as an LDS store and add waits before later
// LDS reads of other buffers; the kernels order these loads themselves (wait
// for the vector-memory counter, then a workgroup barrier, before any read).
// A scalar write of m0 needs one wait state before an LDS-DMA load reads it;
// the hazard recognizer cannot see into an asm block, so the s_nop is written
// out here (the compiler emits the same nop for its own global_load_lds).
__device__ __forceinline__ void dma16(const void* src, const bf16* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds_dst));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}

// Direct global->LDS load of 4 bytes per lane (global_load_lds_dword): lane l
// writes LDS bytes [lds + 4 l, lds + 4 l + 4). Same ordering rules as dma16.
__device__ __forceinline__ void dma4(const void* src, const void* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds_dst));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}

// One 1 KiB slot of a swizzled tile: lane l fills chunk position 64*slot + l,
// fetching the chunk of the source row that the swizzle stores there.
// row_ptr(r) returns the global address of tile row r.
template <int C, typename RowPtr>
__device__ __forceinline__ void dma_slot(bf16* tile, int slot, int lane, RowPtr row_ptr) {
  const int pos = slot * 64 + lane;
  const int r = pos / C;
  const int c = (pos % C) ^ swz<C>(r);
  dma16(row_ptr(r) + 8 * c, tile + slot * 512);
}

// The same direct load with a uniform 64-bit base in SGPRs, a 32-bit per-lane
// byte offset (the global_load "saddr" form) and the LDS destination as a
// uniform byte address: the offset of a slot is fixed for the whole sweep, so
// the per-tile address work is scalar.
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_byte), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Issue priority from progress through a sweep: 3 for its first quarter down
// to 0 for its last. Where several workgroups share a CU the arbiter otherwise
// favours the oldest waves, so the workgroups of one CU finish one after
// another and the CU ends each round with fewer and fewer of them resident;
// with this, a workgroup that is behind gets the issue slots and the CU's
// workgroups advance at one pace.
__device__ __forceinline__ void prio_by_progress(int done, int total, int& cur) {
  const int q = __builtin_amdgcn_readfirstlane(min(3, (4 * done) / max(total, 1)));
  if (q != cur) {
    cur = q;
    if (q == 0)
      __builtin_amdgcn_s_setprio(3);
    else if (q == 1)
      __builtin_amdgcn_s_setprio(2);
    else if (q == 2)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  }
}

// LDS byte address of a __shared__ location (for dma16_s).
__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p);
}

// Byte offset, from the start of the tile's first source row, of the chunk that
// lane l fills in slot `slot` of a swizzled tile with rows of C chunks and
// `row_bytes` between source rows (the mapping of dma_slot).
template <int C>
__device__ __forceinline__ uint32_t slot_offset(int slot, int lane, int row_bytes) {
  const int pos = slot * 64 + lane;
  const int r = pos / C;
  const int c = (pos % C) ^ swz<C>(r);
  return (uint32_t)(r * row_bytes + 16 * c);
}

// Block-mask bits staged in LDS: one 128-row mask row (or column) is at most
// kMaxMaskBlocks entries, so N <= 128 * kMaxMaskBlocks when a block mask is used.
constexpr int kMaxMaskBlocks = 16384;
constexpr int kMaskWords = kMaxMaskBlocks / 32;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace fa

// Workgroup order. The dispatcher hands workgroups to the 8 XCDs round-robin
// (workgroup i to XCD i mod 8) and each XCD has its own L2. Interleaved order
// (HEAD_MAJOR false): head i mod BH, block i / BH, so block 0 of every head
// goes first; with B*H a multiple of 8 all of one head's blocks still land on
// one XCD. Head-major order (HEAD_MAJOR true, B*H a multiple of 8): workgroup
// i = 8j + x takes head x + 8*(j / nblk) and block j mod nblk, so each XCD
// works through its heads one after another and the tiles one head's blocks
// re-read stay in that XCD's L2 while in use; it helps when the blocks of a
// head read different tiles (a block mask) and costs the global largest-first
// order that causal launches want. Callers map block 0 to their largest block.
struct WgCoord {
  int bh;
  int blk;
};
template <bool HEAD_MAJOR>
__device__ __forceinline__ WgCoord wg_coord(int i, int BH, int nblk) {
  if (HEAD_MAJOR && (BH & 7) == 0) {
    const int j = i >> 3;
    return {(i & 7) + 8 * (j / nblk), j % nblk};
  }
  return {i % BH, i / BH};
}
