// Host-side launch helper shared by the kernel files.
//
// A kernel dispatch carries its grid as a 32-bit count of work-items per
// dimension, and a 1-D launch of 2^32 work-items or more is cut short
// without an error: on gfx950 under ROCm 7.2, a launch of 2^26 + 1
// workgroups of 64 lanes reported success and ran one workgroup.  Every
// launcher therefore splits its grid into chunks of whole units (heads for
// the kernels that tile heads, blocks of rows for the row-wise kernels), each
// launch at most kMaxLaunchItems work-items, and moves its base pointers per
// chunk; the kernels see a smaller problem of the same layout.  The cap of
// 2^31 also keeps every workgroup and lane index of one launch inside int32.
#pragma once

#include <algorithm>
#include <cstdint>

namespace fa {

constexpr int64_t kMaxLaunchItems = int64_t(1) << 31;

// Returned (instead of a hipError_t, which is >= 0) when a single unit's
// grid alone exceeds the cap; nothing has been launched.  The C ABI reports
// it as FA_ERR_SHAPE.
constexpr int kErrGridTooLarge = -1;

inline bool unit_fits(int64_t items_per_unit) { return items_per_unit <= kMaxLaunchItems; }

// Calls launch(first, count) for consecutive chunks covering units [0, units),
// each of at most kMaxLaunchItems / items_per_unit units; returns the first
// non-zero status.  One chunk (the common case) is one call.
template <typename F>
int launch_in_chunks(int64_t units, int64_t items_per_unit, F&& launch) {
  if (!unit_fits(items_per_unit)) return kErrGridTooLarge;
  const int64_t per = kMaxLaunchItems / items_per_unit;
  for (int64_t u0 = 0; u0 < units; u0 += per) {
    const int e = launch(u0, std::min(per, units - u0));
    if (e != 0) return e;
  }
  return 0;
}

}  // namespace fa
