// Argument checks for the attention C ABI.  Pure C++ with no HIP dependency,
// so that it can be compiled and sanitised on a host compiler by itself.
// Every check runs before anything is enqueued on a stream.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "../../include/fa.h"

namespace fa {

struct Shape {
  int64_t B, H, N, d;
  bool empty() const { return B == 0 || H == 0 || N == 0; }
  // Elements of one [B][H][N][d] tensor / one [B][H][N] row vector.
  int64_t elems() const { return B * H * N * d; }
  int64_t rows() const { return B * H * N; }
};

// Largest tensor accepted: 2^40 elements keeps every byte offset and
// per-head offset far inside int64.  Grids are cut into launches of at most
// 2^31 work-items by the launchers, so the total size sets no grid limit.
constexpr int64_t kMaxElems = int64_t(1) << 40;

inline fa_status check_shape(const Shape& s, bool bf16) {
  if (s.B < 0 || s.H < 0 || s.N < 0 || s.d <= 0) return FA_ERR_SHAPE;
  if (bf16) {
    if (s.d != 64 && s.d != 128) return FA_ERR_UNSUPPORTED;
  } else if (s.d > 128) {
    return FA_ERR_UNSUPPORTED;
  }
  if (s.empty()) return FA_OK;
  // Row indices inside the kernels are 32-bit.
  if (s.N > (int64_t(1) << 31) - 1) return FA_ERR_SHAPE;
  // The bf16 kernels address one head of one tensor with 32-bit byte offsets
  // (including a tile of rows past the end): at most 2 GiB per head.
  if (bf16 && (s.N + 128) * s.d * 2 > (int64_t(1) << 31) - 1) return FA_ERR_SHAPE;
  // Overflow-safe product check.
  const int64_t lim = kMaxElems;
  if (s.B > lim || s.H > lim / s.B) return FA_ERR_SHAPE;
  const int64_t bh = s.B * s.H;
  if (s.N > lim / bh) return FA_ERR_SHAPE;
  if (s.d > lim / (bh * s.N)) return FA_ERR_SHAPE;
  return FA_OK;
}

inline fa_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
  return FA_OK;
}

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

struct Span {
  const void* p;
  size_t bytes;
};

inline bool overlap(const Span& a, const Span& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  if (a.bytes == 0 || b.bytes == 0) return false;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output must be disjoint from every input and from the other outputs.
inline fa_status check_alias(std::initializer_list<Span> inputs,
                             std::initializer_list<Span> outputs) {
  for (auto o = outputs.begin(); o != outputs.end(); ++o) {
    for (const Span& i : inputs)
      if (overlap(*o, i)) return FA_ERR_ALIAS;
    for (auto o2 = o + 1; o2 != outputs.end(); ++o2)
      if (overlap(*o, *o2)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

inline fa_status check_ptrs(std::initializer_list<const void*> ptrs, size_t align) {
  for (const void* p : ptrs)
    if (p == nullptr) return FA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned(p, align)) return FA_ERR_ALIGN;
  return FA_OK;
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of the backward: one fp32 per query row for D = rowsum(dO * O).
inline size_t bwd_workspace_bytes(const Shape& s, bool bf16) {
  if (check_shape(s, bf16) != FA_OK) return static_cast<size_t>(-1);
  if (s.empty()) return 0;
  return round_up(static_cast<size_t>(s.rows()) * sizeof(float), 256);
}

// Split-KV forward: n_split contiguous ranges of whole key tiles of `tile`
// keys, at least one tile per range.
inline int64_t split_max(const Shape& s, int64_t tile) {
  if (check_shape(s, true) != FA_OK) return -1;
  if (s.empty()) return 0;
  return (s.N + tile - 1) / tile;
}

// Most partial results a merge takes: the kernels count parts in int32 (in
// steps of 8), and the split forward makes fewer than 2^24 ranges.
constexpr int64_t kMaxParts = int64_t(1) << 24;

// n_split partial tensors of the shape: the count must be in [1, kMaxParts]
// and the partials must stay inside the size limit.
inline fa_status check_parts(const Shape& s, int64_t n_split) {
  if (n_split < 1 || n_split > kMaxParts) return FA_ERR_SHAPE;
  if (s.empty()) return FA_OK;
  if (n_split > kMaxElems / s.elems()) return FA_ERR_SHAPE;
  return FA_OK;
}

inline fa_status check_workspace(const void* ws, size_t bytes, size_t need) {
  if (need == 0) return FA_OK;
  if (ws == nullptr) return FA_ERR_NULL;
  if (bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}

#define FA_TRY(expr)                      \
  do {                                    \
    const fa_status fa_try_s_ = (expr);   \
    if (fa_try_s_ != FA_OK) return fa_try_s_; \
  } while (0)

}  // namespace fa
