// Merge of split-KV partial results.  For one query row, key range p gave a
// normalised output O_p = sum_{j in p} e^{s_j - LSE_p} v_j and LSE_p =
// ln sum_{j in p} e^{s_j}.  The rescale identity of the star-observatory
// fable (ckw19810413.github.io, section "兩大核心魔法": e^{x-m_new} =
// e^{x-m_old} e^{m_old-m_new}) gives the full row:
//   LSE = m + ln sum_p e^{LSE_p - m}          (m = max_p LSE_p)
//   O   = sum_p e^{LSE_p - LSE} O_p
// Order of the ranges does not matter (算珠楼的掌簿人, hespethorn.github.io,
// section 四: accounts kept separately combine without conflict).
//
// Memory-bound: per row it reads nsplit * (4d + 4) bytes and writes 2d + 4.
// D/4 lanes per row, 16 bytes per lane per partial, eight partials' loads in
// flight at a time; the LSEs of a row are read by all of its lanes (one
// cache line).  A range whose LSE is -inf
// (no key) contributes nothing, whatever its O_p holds; a row with no range
// holding a key gets O = 0 and LSE = -inf.
#include "device_common.h"
#include "launch_chunks.h"

namespace fa {
namespace {

// `rows` rows of this launch, each part `part_stride` rows apart.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part,
                                                    int nsplit, int64_t rows,
                                                    int64_t part_stride,
                                                    uint16_t* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int LPR = D / 4;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per block
  constexpr int CH = 8;               // parts loaded together (independent loads in flight)
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int col = (tid % LPR) * 4;
  if (row >= rows) return;

  // One pass over the parts with a running reference m (the same identity
  // applied part by part): acc = sum_p e^{LSE_p - m} O_p, den = sum_p
  // e^{LSE_p - m}; when m grows, both are multiplied by e^{m_old - m_new}.
  float m = -INFINITY, den = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int p0 = 0; p0 < nsplit; p0 += CH) {
    float lp[CH];
    f32x4 op[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int p = p0 + c;
      lp[c] = p < nsplit ? lse_part[p * part_stride + row] : -INFINITY;
      op[c] = p < nsplit
                  ? *reinterpret_cast<const f32x4*>(o_part + (p * part_stride + row) * D + col)
                  : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float mc = m;
#pragma unroll
    for (int c = 0; c < CH; ++c) mc = fmaxf(mc, lp[c]);
    if (mc == -INFINITY) continue;                     // no live part so far
    const float r = m == -INFINITY ? 0.0f : __expf(m - mc);
    den *= r;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= r;
    m = mc;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lp[c] == -INFINITY) continue;                // a part with no key: O_p not used
      const float w = __expf(lp[c] - m);
      den += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, op[c][e], acc[e]);
    }
  }
  float lse_row = -INFINITY;
  if (den > 0.0f) {
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= inv;
    lse_row = m + __logf(den);
  }
  u32x2 w;
  w[0] = pack_bf16x2(acc[0], acc[1]);
  w[1] = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<u32x2*>(o + row * D + col) = w;
  if (col == 0) lse[row] = lse_row;
}

template <int D>
int launch_merge(const float* o_part, const float* lse_part, int nsplit, int64_t rows,
                 uint16_t* o, float* lse, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  // Chunks of whole blocks of RPB rows; each part keeps its stride of `rows`.
  return launch_in_chunks((rows + RPB - 1) / RPB, 256, [&](int64_t b0, int64_t nb) {
    const int64_t r0 = b0 * RPB, nr = std::min(nb * RPB, rows - r0);
    hipLaunchKernelGGL(merge_kernel<D>, dim3((unsigned)nb), dim3(256), 0, stream,
                       o_part + r0 * D, lse_part + r0, nsplit, nr, rows, o + r0 * D, lse + r0);
    return (int)hipGetLastError();
  });
}

}  // namespace

int launch_merge_bf16(const float* o_part, const float* lse_part, int nsplit, int64_t rows,
                      int64_t d, void* o, float* lse, hipStream_t stream) {
  auto* o16 = static_cast<uint16_t*>(o);
  return d == 128 ? launch_merge<128>(o_part, lse_part, nsplit, rows, o16, lse, stream)
                  : launch_merge<64>(o_part, lse_part, nsplit, rows, o16, lse, stream);
}

}  // namespace fa
