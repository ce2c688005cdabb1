// Device helpers shared by the gfx950 attention kernels: vector types, the
// bf16 matrix-core instruction, and small load/convert utilities.
//
// Matrix-core layout of the dK/dV kernel (v_mfma_f32_32x32x16_bf16, one wave of
// 64 lanes; l = lane, g = l / 32):
//   A operand (32 x 16, row r, k):  lane l holds row r = l % 32, the 8 values
//                                   of its k-group g.
//   B operand (16 x 32, k, col c):  lane l holds col c = l % 32, the 8 values
//                                   of its k-group g.
//   C/D (32 x 32 fp32):             lane l, element i (0..15) holds
//                                   row 8*(i/4) + 4*g + (i%4), col l % 32.
// Because A and B use the same lane/k-group convention, a contraction is
// correct whenever both operands enumerate the same k indices in the same
// (group, element) order; the hardware's internal order of k does not matter.
//
// The forward and the dQ pass use the 16 x 16 x 32 form
// (v_mfma_f32_16x16x32_bf16; g = l / 16):
//   A operand (16 x 32):  lane l holds row l % 16, the 8 values of k-group g.
//   B operand (32 x 16):  lane l holds col l % 16, the 8 values of k-group g.
//   C/D (16 x 16 fp32):   lane l, element i (0..3) holds row 4*g + i, col l % 16.
// It does the same work per cycle as the 32 x 32 form at its peak, and on
// operands with random mantissas (bf16 data of unit scale) it sustains a
// higher rate on this part: 1.98-2.03 PF/s against 1.76-1.77 PF/s, two waves
// per SIMD, independent instructions (measured).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Round-to-nearest-even fp32 -> bf16 pair (lowered to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 p;
  p[0] = static_cast<__bf16>(a);
  p[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte LDS read of 8 bf16 (address 16-byte aligned).
__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resources: loads through them return 0 past `bytes`, which covers
// the ragged last tile without branches.  The base must be wave-uniform;
// byte offsets are 32-bit, so one resource spans at most 4 GiB (the API
// limits one head of one tensor to 2 GiB).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit data format (CDNA)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Waits until every vector-memory load this wave issued has completed,
// including direct buffer->LDS loads.
// (s_waitcnt vmcnt(0): vmcnt bits 0 in [3:0] and [15:14], expcnt 7 in [6:4],
// lgkmcnt 15 in [11:8].  The builtin, unlike inline assembly, is seen by the
// compiler's own wait insertion.)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float buf_loadf(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Maps the hardware workgroup id to a logical tile id so that consecutive
// logical ids (the tiles of one head) run on the same XCD: workgroups are
// dealt to the 8 XCDs round-robin, and each XCD has its own L2, so a head's
// streamed tiles are fetched into one L2 and reused there.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int x = wg & 7, idx = wg >> 3;
  const int base = nwg >> 3, rem = nwg & 7;
  return x * base + (x < rem ? x : rem) + idx;
}

// acc + a.lo + a.hi for the two bf16 values packed in the dword a (one
// v_dot2 against (1, 1); the products are exact).
__device__ __forceinline__ float add_bf16x2(uint32_t a, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

// Lanes l and l ^ 32 exchange a value with v_permlane32_swap: called with
// the same register twice, the two results hold x[l % 32] and x[l % 32 + 32]
// in every lane (a VALU op, no LDS round trip).
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes of one
// column of a 16 x 16 accumulator): v_permlane16_swap exchanges lanes l and
// l ^ 16 the way v_permlane32_swap exchanges l and l ^ 32.
__device__ __forceinline__ float max_across_quarters(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max_across_halves(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

__device__ __forceinline__ float sum_across_quarters(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return sum_across_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

}  // namespace fa
