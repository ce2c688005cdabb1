// Row-major bf16 tiles in LDS, filled by direct buffer->LDS loads and read
// either along rows (16-byte reads) or across rows (transposing reads).
//
// Layout.  A tile holds rows of D bf16 values (2*D bytes, no padding).  Each
// row is a sequence of 16-byte chunks; logical chunk c of row r is stored at
// physical chunk c ^ swz<D>(r).  LDS has 64 banks of 4 bytes; the swizzle
// keeps both read patterns below conflict-free (SQ_LDS_BANK_CONFLICT is 0
// for the kernel that uses these tiles).  It was chosen for groups of 16
// consecutive lanes, which 16-byte reads are not served in (row-segment
// tiles below), but on these patterns the measured groups see distinct
// banks as well:
//   - row operands: 16 consecutive rows, one logical chunk each.  With
//     D = 128 a row spans all 64 banks and the bank group is the physical
//     chunk, so swz must take 16 distinct values on 16 consecutive rows;
//     with D = 64 two rows share the banks (row parity picks the half), so
//     swz must be distinct on the 8 rows of each parity.
//   - transposed operands: 4 consecutive rows (from a multiple of 4), the 4
//     chunks of one 32-column block each: the 4 rows (per parity, D = 64)
//     must land on different 4-chunk blocks.
//   D = 128: swz(r) = 4 (r & 3) + ((r >> 2) & 3)
//   D = 64:  swz(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3)
// Loads.  A direct buffer->LDS load writes lane L's 16 bytes at LDS address
// M0 + 16 L whatever global address the lane read, so the swizzle is applied
// on the global side: the lane that fills physical chunk p of row r reads
// logical chunk p ^ swz(r) of that row.  Reads past the end of the buffer
// resource return zeros.
//
// Transposing read.  ds_read_b64_tr_b16 works on groups of 16 lanes: source
// lane 4a + b supplies the address of 4 consecutive bf16 values, and result
// lane i receives element i % 4 of source lanes i/4, i/4 + 4, i/4 + 8 and
// i/4 + 12.  Two such reads (tr_read_off, tr_read2) give lane l (column
// cbase + l % 32, k-group g = l / 32) the values of rows
// {4g..4g+3, 8+4g..8+4g+3} of a 16-row step in that column: exactly the
// operand a 32x32x16 matrix-core instruction needs when its contraction
// index runs along the tile's rows and the other operand comes from score
// accumulators.
#pragma once

#include "device_common.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "tile widths of 64 or 128 bf16");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One direct buffer->LDS load of 16 bytes per lane: lane L's bytes land at
// LDS byte address lds + 16 L (lds wave-uniform).  Issued as inline assembly
// so that the compiler does not order later LDS reads of *other* buffers
// behind it; completion is awaited explicitly (wait_vmem) before the barrier
// that publishes the tile.  M0 is saved and restored around the load.
// The byte offset is voff (per lane) + soff (wave-uniform).
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint32_t voff, uint32_t lds,
                                          uint32_t soff = 0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(lds), "s"(soff)
      : "memory");
}

// The same with 4 bytes per lane: lane L's dword lands at lds + 4 L.
__device__ __forceinline__ void lds_dma4(rsrc_t r, uint32_t voff, uint32_t lds,
                                         uint32_t soff = 0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dword %1, %2, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(lds), "s"(soff)
      : "memory");
}

// ---------------------------------------------------------------------------
// Swizzled tiles with per-lane offset tables.  When a tile is loaded one
// instruction at a time (interleaved with other work) and read through
// per-lane pointers computed once, neither side does address arithmetic in
// the loop.
//
// Direct loads: wave w of NW issues instructions u = 0, 1, ... covering
// physical chunks (w + u NW) * 64 + lane.  Consecutive instructions of a wave
// are NW*64/(D/8) rows apart, a multiple of the swizzle period (16 rows), so
// the per-lane source offset is the same for every u (tile_dma_voff) and the
// rest of the address is wave-uniform.
template <int D, int NW>
__device__ __forceinline__ uint32_t tile_dma_voff(int wave, int lane) {
  constexpr int NC = D / 8;
  const int lin = wave * 64 + lane, row = lin / NC, phys = lin % NC;
  return (uint32_t)((row * D + ((phys ^ swz<D>(row)) << 3)) * 2);
}
// Instruction u of this wave: `tile_lds` is the tile's LDS byte address and
// `row0_bytes` the byte offset of the tile's first row in `src` (both
// wave-uniform).
template <int D, int NW>
__device__ __forceinline__ void tile_dma(uint32_t tile_lds, rsrc_t src, uint32_t voff,
                                         uint32_t row0_bytes, int wave, int u) {
  constexpr int RSTEP = NW * 64 / (D / 8);
  static_assert(RSTEP % 16 == 0, "whole swizzle periods between instructions");
  lds_dma16(src, voff, tile_lds + (uint32_t)((wave + u * NW) * 1024),
            row0_bytes + (uint32_t)(u * RSTEP * D * 2));
}
// Element offset of this lane's row operand at k-step kk in rows 0..31 (row
// lane % 32, logical chunk 2 kk + lane / 32).  32-row block kb adds kb*32*D.
template <int D>
__device__ __forceinline__ int row_read_off(int lane, int kk) {
  const int r = lane & 31, c = 2 * kk + (lane >> 5);
  return r * D + ((c ^ swz<D>(r)) << 3);
}
// Element offset of this lane's half-h transposing read of 32-column block
// cb in rows 0..15: source rows 4 g + a + 8 h (g = (lane / 16) / 2, a =
// (lane % 16) / 4), columns 32 cb + 16 ((lane / 16) % 2) + 4 (lane % 4)
// ..+3.  16-row step t adds t*16*D.
template <int D>
__device__ __forceinline__ int tr_read_off(int lane, int cb, int h) {
  const int i16 = lane & 15, q = lane >> 4;
  const int a = i16 >> 2, b = i16 & 3, g = q >> 1;
  const int col = cb * 32 + 16 * (q & 1) + 4 * b;
  const int r = 4 * g + a + 8 * h;
  return r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 7);
}
// The transposed operand from the two halves' addresses.
__device__ __forceinline__ bf16x8 tr_read2(const uint16_t* p1, const uint16_t* p2) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p1));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p2));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 w = {l2[0], l2[1], h2[0], h2[1]};
  return as_bf16x8(w);
}

// ---------------------------------------------------------------------------
// Row-segment tiles.  R rows of D bf16 values in 1 KB blocks of 16 rows x 32
// values: block (r16, c32) sits at byte (r16 * D/32 + c32) * 1024 and holds
// the 64 bytes of its row rho at byte 64 rho, as four 16-byte pieces.  One
// direct load fills one block, lanes 4 rho .. 4 rho + 3 reading the 64
// contiguous source bytes of row rho: the load path runs at full rate only
// when every four consecutive lanes read one contiguous 64-byte segment
// (a load whose lanes cover 32 rows x 32 bytes, the order of a matrix-core
// operand, runs at a quarter of it; two lanes per row at a half).  Piece p
// of row rho sits at position p ^ seg_swz(rho).
// LDS service order (measured with SQ_LDS_BANK_CONFLICT on synthetic lane
// patterns): a 16-byte read (ds_read_b128) is served in four groups of 16
// lanes, each group the lanes of one half-wave whose lane bits 2, 3 and 4
// have the same parity, and a group is conflict-free when its 16 reads fall
// on 16 different 4-bank groups; 8-byte transposing reads showed no
// conflicts on these tiles.  Flipping bit 1 of the piece by bit 2 of the row
// makes both the row-operand reads and the transposing reads below
// conflict-free (without a swizzle, or with one chosen for 16 consecutive
// lanes, every row-operand read costs a second pass).
__host__ __device__ constexpr int seg_swz(int rho) { return 2 * ((rho >> 2) & 1); }
template <int D, int NW>
__device__ __forceinline__ uint32_t seg_dma_voff(int wave, int lane) {
  constexpr int C32 = D / 32;
  static_assert(NW % C32 == 0, "whole 16-row steps between a wave's instructions");
  const int rho = lane >> 2, pos = lane & 3;
  const int p = pos ^ seg_swz(rho);
  const int row = (wave / C32) * 16 + rho, col = (wave % C32) * 32 + p * 8;
  return (uint32_t)((row * D + col) * 2);
}
// Instruction u of wave `wave` fills block wave + u NW of the tile at LDS
// byte address `tile_lds`; `row0_bytes` is the source offset of its row 0.
template <int D, int NW>
__device__ __forceinline__ void seg_dma(uint32_t tile_lds, rsrc_t src, uint32_t voff,
                                        uint32_t row0_bytes, int wave, int u) {
  constexpr int USTEP = (NW / (D / 32)) * 16 * D * 2;
  lds_dma16(src, voff, tile_lds + (uint32_t)((wave + u * NW) * 1024),
            row0_bytes + (uint32_t)(u * USTEP));
}
// Operands of the 16 x 16 x 32 instruction (device_common.h).
// Row operand: for 16-row block kb and 32-column k-step kk, lane L takes
// the 8 values of row 16 kb + L % 16 at columns 32 kk + 8 (L / 16) ..+7.
__device__ __forceinline__ uint32_t seg_rowop16_base(int lane) {
  const int rho = lane & 15, g = lane >> 4;
  return (uint32_t)(64 * rho + 16 * (g ^ seg_swz(rho)));
}
template <int D>
__host__ __device__ constexpr int seg_rowop16_imm(int kb, int kk) {
  return (kb * (D / 32) + kk) * 1024;
}
// Transposed operand: for 32-row step t and 16-column block cb, lane L
// (column 16 cb + L % 16, k-group g = L / 16) takes rows 32 t + 4 g + 0..3
// (elements 0..3) and 32 t + 16 + 4 g + 0..3 (elements 4..7) of its column:
// the key order of two 16 x 16 score accumulators of 16 keys each.  Source
// lane 4 a + b of group g addresses row 4 g + a of the block, columns
// 16 (cb & 1) + 4 b ..+3.  Base for blocks of parity e.
__device__ __forceinline__ uint32_t seg_trop16_base(int lane, int e) {
  const int i16 = lane & 15, g = lane >> 4, a = i16 >> 2, b = i16 & 3;
  const int rho = 4 * g + a;
  return (uint32_t)(64 * rho + 16 * ((2 * e + (b >> 1)) ^ seg_swz(rho)) + 8 * (b & 1));
}
template <int D>
__device__ __forceinline__ bf16x8 seg_trop16_read(const uint8_t* lanebase, int t, int cb) {
  const uint8_t* p = lanebase + (2 * t * (D / 32) + cb / 2) * 1024;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p + (D / 32) * 1024));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 w = {l2[0], l2[1], h2[0], h2[1]};
  return as_bf16x8(w);
}

}  // namespace fa
