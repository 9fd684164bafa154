// LDS tile helpers for the bf16 MFMA kernels (gfx950).
//
// A tile holds up to 64 token rows of one head; each row is 256 bytes (128 bf16,
// a 64-wide row uses the first half) split into 16 chunks of 16 bytes.  Chunk c
// of row r is stored at chunk position c ^ swz(r), swz(r) = 4*(r%4) + (r/4)%4.
// With this swizzle both access patterns the kernels use are free of LDS bank
// conflicts:
//   * row reads: 16 lanes read the same logical chunk of 16 consecutive rows
//     (an MFMA operand whose contraction index runs along the row) -- swz is a
//     bijection on any 16 consecutive rows starting at a multiple of 16;
//   * transposed reads (ds_read_b64_tr_b16): 16 lanes read 4 consecutive rows x
//     4 consecutive chunks -- the row's low bits move the chunk's high bits, so
//     the 16 chunks land in 16 distinct positions.
// Tiles are filled with direct global->LDS loads (global_load_lds_dwordx4): one
// wave instruction writes 1 KB = 4 rows, lane i the 16 bytes at offset 16*i; the
// swizzle is applied on the global side by choosing which chunk lane i fetches.
#pragma once

#include "pa_common.h"

namespace pa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_cvoid;

constexpr int kRowBytes = 256;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ int tile_byte(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// Block -> (work item, head).  Workgroups are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8).  When the head count is a multiple of 8, XCD x
// walks its heads x, x+8, ... one after the other, each over all work items in
// the given (longest-first) order, so the blocks in flight on an XCD share one
// head's K/V (or Q/dO) rows in that XCD's L2.  Otherwise heads vary fastest.
__device__ __forceinline__ void block_work(int b, int H, int nwork, int* work, int* h) {
  if ((H & 7) == 0) {
    const int xcd = b & 7, slot = b >> 3;
    const int hg = slot / nwork;
    *work = slot - hg * nwork;
    *h = xcd + 8 * hg;
  } else {
    *work = b / H;
    *h = b - *work * H;
  }
}

// Wave-uniform index of the calling wave inside its workgroup (kept in an SGPR).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Copy token rows row0 .. row0 + NROWS - 1 of head `h` (tensor [n][H][D] bf16,
// `rs` elements between tokens) into an LDS tile.  Rows at or past n re-read
// row n - 1; callers mask those positions.  NW waves share the work.
template <int D, int NROWS, int NW>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ g, size_t rs, int hoff,
                                           int row0, int n, char* tile, int wv, int lane) {
  static_assert(NROWS % 4 == 0, "tile rows come in groups of 4");
  const int p = lane & 15, rl = lane >> 4;  // physical chunk, row within the 4-row group
  if (row0 + NROWS <= n) {
    // Every row exists: a wave-uniform row base plus a per-lane byte offset
    // (row r = 4*blk + rl has swz(r) = 4*rl + blk%4).
#pragma unroll
    for (int blk = wv; blk < NROWS / 4; blk += NW) {
      int c = p ^ (4 * rl + (blk & 3));
      if (D == 64) c &= 7;  // 64-wide rows use chunks 0..7; other slots get a spare copy
      const uint32_t lane_off = (uint32_t)(((size_t)rl * rs + hoff + c * 8) * 2);
      const char* base = (const char*)(g + (size_t)(row0 + 4 * blk) * rs);
      __builtin_amdgcn_global_load_lds((global_cvoid*)(base + lane_off),
                                       (lds_void*)(tile + blk * 1024), 16, 0, 0);
    }
  } else {
    // Tail tile: rows at or past n re-read row n - 1 (callers mask them).
#pragma unroll
    for (int blk = wv; blk < NROWS / 4; blk += NW) {
      const int r = blk * 4 + rl;
      int c = p ^ swz(r);
      if (D == 64) c &= 7;
      const int gr = min(row0 + r, n - 1);
      const uint16_t* src = g + (size_t)gr * rs + hoff + c * 8;
      __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)(tile + blk * 1024), 16, 0,
                                       0);
    }
  }
}

// Copy `count` (<= 64) consecutive 32-bit values starting at src[i0] (clamped to
// src[n - 1]) into LDS; one wave instruction, lane i writes dst[i].
__device__ __forceinline__ void stage_words(const void* __restrict__ src, int i0, int n,
                                            char* dst, int lane) {
  const int i = min(i0 + lane, n - 1);
  __builtin_amdgcn_global_load_lds((global_cvoid*)((const uint32_t*)src + i), (lds_void*)dst, 4,
                                   0, 0);
}

// A seq id no allowed pair carries (allowed pairs have ids >= 0); read, never written.
__device__ int32_t kNoId = -1;

// Copy the 64 seq ids ids[i0 .. i0+63] into LDS; positions at or past n get -1,
// so a tail tile needs no separate bounds test (one wave instruction).
__device__ __forceinline__ void stage_ids(const int32_t* __restrict__ ids, int i0, int n,
                                          char* dst, int lane) {
  const int i = i0 + lane;
  const int32_t* src = i < n ? ids + i : &kNoId;
  __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)dst, 4, 0, 0);
}

// Direct global->LDS loads issued from inline assembly.  The compiler does
// not see these LDS writes, so it cannot answer them with conservative
// vmcnt(0) waits in front of unrelated LDS reads (it did with the builtins
// once three buffers of each kind were in flight); every use is ordered by
// explicit vmcnt waits and barriers instead.  A kernel that uses them issues
// no other LDS-DMA (they set M0 themselves).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// raw buffer descriptor over `bytes` bytes from `base` (range-checked loads)
__device__ __forceinline__ u32x4_t raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// 16 bytes per lane from rsrc at byte offset voff to LDS (lane i at lds + 16 i)
__device__ __forceinline__ void dma_b128(u32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds) : "memory");
}

// 4 bytes per lane from the lane's address to LDS (lane i at lds + 4 i)
__device__ __forceinline__ void dma_b32(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               ::"v"(src), "s"(lds) : "memory");
}

// 4 bytes per lane from rsrc at byte offset voff to LDS (lane i at lds + 4 i).
// Measured cheaper than dma_b32 in the paired kernels (the global form slowed
// the other group's MFMA phase while in flight); reads past the descriptor's
// range return 0, so callers keep dma_b32 where a tail needs another fill.
__device__ __forceinline__ void dma_b32_buf(u32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds) : "memory");
}

// Class byte of tile pair `idx`, fetched as the aligned 32-bit word that holds
// it: a uniform word address becomes a scalar (SMEM) load, which -- unlike a
// vector byte load -- does not make the wave wait behind its outstanding
// direct-to-LDS loads of the next stage.  The class array is padded to a
// multiple of 256 bytes, so the word never leaves the allocation.
__device__ __forceinline__ int tile_class_at(const uint8_t* __restrict__ cls, size_t idx) {
  const uint32_t w = ((const uint32_t*)cls)[idx >> 2];
  return (int)((w >> (8 * (idx & 3))) & 0xFFu);
}

// A uniform 32-bit load issued where it stands (s_load_dword from inline
// assembly: the compiler would otherwise sink it to its first use) and landed
// by sload_wait, which the value is tied to, so nothing reads it earlier.  The
// compiler does not count this load; its own lgkmcnt waits stay correct (they
// can only wait longer while it is in flight).  `p` must be 4-byte aligned.
__device__ __forceinline__ int32_t sload_issue(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ void sload_wait(int32_t& v) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v)::"memory");
}
__device__ __forceinline__ void sload_wait2(int32_t& a, int32_t& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(a), "+s"(b)::"memory");
}

// Wait for this wave's outstanding direct-to-LDS loads.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

__device__ __forceinline__ bf16x8 lds_row8(const char* tile, int byte) {
  return *(const bf16x8*)(tile + byte);
}

__device__ __forceinline__ i16x4 lds_tr4(const char* tile, int byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tile + byte));
}

__device__ __forceinline__ bf16x8 join8(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v;
  v.lo = lo;
  v.hi = hi;
  return __builtin_bit_cast(bf16x8, v);
}

// Per-lane byte offsets (within a tile) of the MFMA operand reads.
//
// Row operand (32x32x16 A or B, contraction along the row): lane l reads row
// 32*mb + (l % 32), logical chunk 2*kk + l/32.  The swizzle of such a row does
// not depend on mb, so row_off(kk) + 8192*mb is the byte offset.
__device__ __forceinline__ int row_off(int lane, int kk) {
  const int r = lane & 31;
  return r * kRowBytes + (((2 * kk + (lane >> 5)) ^ swz(r)) << 4);
}

// Transposed operand via ds_read_b64_tr_b16: the 16 lanes of a group together
// fetch rows k0 .. k0+3 (4 bytes... 8 bytes per lane) and return, to lane L of
// the group, the 4 values of column m0 + L at rows k0 .. k0+3.  For the 32x32x16
// A operand (m = l % 32, 8 contraction slots per lane) with the contraction
// slots mapped to rows {16kb + 4h + 0..3, 16kb + 8 + 4h + 0..3} (h = l / 32),
// lane l supplies row 16kb + 4h + (L/4) (+8 for the second read) and columns
// 32*db + 16*((l/16)%2) + 4*(L%4).  The swizzle of those rows does not depend
// on kb, so tr_off(db, s) + 4096*kb is the byte offset (s = first/second read).
__device__ __forceinline__ int tr_off(int lane, int db, int s) {
  const int L = lane & 15, h = lane >> 5, gm = (lane >> 4) & 1;
  const int row = 4 * h + (L >> 2) + 8 * s;
  const int col = 32 * db + 16 * gm + 4 * (L & 3);  // element index in the row
  return row * kRowBytes + (((col >> 3) ^ swz(row)) << 4) + ((col & 7) << 1);
}

// Lane-constant bases of the same offsets.  Both offset families only differ
// per instruction in bits that the base keeps free or XORs, so
//   row_off(lane, kk)   == row_base(lane) ^ (32 * kk)
//   tr_off(lane, db, s) == (tr_base(lane) ^ (64 * db + 32 * s)) + 2048 * s
// (the row swizzle term of 16*chunk XORs into bits 4..7; rows sit in bits >= 8).
// One v_xor per offset keeps only two address registers live.
__device__ __forceinline__ int row_base(int lane) { return row_off(lane, 0); }
__device__ __forceinline__ int tr_base(int lane) { return tr_off(lane, 0, 0); }
__device__ __forceinline__ int row_at(int base, int kk) { return base ^ (32 * kk); }
__device__ __forceinline__ int tr_at(int base, int db, int s) {
  return (base ^ (64 * db + 32 * s)) + 2048 * s;
}

}  // namespace pa
