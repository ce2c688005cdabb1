// fp32 attention kernels: plain FMA arithmetic, natural exp, 8-query by 8-key
// tiles, one wave per workgroup.  They follow the tiled recurrence with the
// blocks of the fable of the 64 merchants (算珠楼的掌簿人, fable section 二: 64
// rows cut into 8 stacks of 8) and take the head dims the matrix-core fp32
// kernels (attn_f32_mfma.hip, d = 64 and 128) do not.
//
// Forward, per query row (账房先生的奔命, section 六; rescale identity of the
// star-observatory fable page, section "兩大核心魔法"):
//   m' = max(m, rowmax S_b);  a = exp(m - m');  p = exp(S_b - m')
//   l  = a l + rowsum p;      U = a U + p V_b;  m = m'
// then O = U / l and LSE = m + ln l.
// Backward (账房先生的奔命, section 七: P recomputed from Q, K and LSE):
//   P = exp(s q.k - LSE),  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * O)
//   dV = P^T dO,  dK = s dS^T Q,  dQ = s dS K.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch_chunks.h"

namespace fa {
namespace {

constexpr int T = 8;        // rows per tile (queries and keys)
constexpr int DMAX = 128;   // largest head dim of the fp32 path
constexpr int CPT = DMAX / T;  // columns per thread

// One thread's share of a T-row tile of a [N][d] matrix: row t / 8, columns
// t % 8 + 8u (no division by the runtime d; eight threads read 32
// consecutive bytes).  Rows at or past N are zero.  fetch_tile loads it into
// registers, put_tile writes it to a [T][DMAX] LDS tile, so that the next
// tile's loads are in flight while the current tile is used.
struct TileRegs {
  float x[CPT];
};

__device__ __forceinline__ void fetch_tile(TileRegs& tr, const float* src, int r0, int N,
                                           int d) {
  static_assert(T * T == 64, "one wave: T rows of T threads");
  const int r = threadIdx.x >> 3, c0 = threadIdx.x & 7;
  const bool live = r0 + r < N;
  const float* row = src + (int64_t)(live ? r0 + r : 0) * d;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = c0 + T * u;
    tr.x[u] = (live && c < d) ? row[c] : 0.0f;
  }
}

__device__ __forceinline__ void put_tile(float (*dst)[DMAX], const TileRegs& tr, int d) {
  const int r = threadIdx.x >> 3, c0 = threadIdx.x & 7;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = c0 + T * u;
    if (c < d) dst[r][c] = tr.x[u];
  }
}

__device__ __forceinline__ void load_tile(float (*dst)[DMAX], const float* src, int r0, int N,
                                          int d) {
  TileRegs tr;
  fetch_tile(tr, src, r0, N, d);
  put_tile(dst, tr, d);
}

__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  return fmaxf(x, __shfl_xor(x, 4));
}

__device__ __forceinline__ float group8_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x + __shfl_xor(x, 4);
}

// Dot products of two rows of d floats with four partial sums: element c
// goes to sum c % 4 (in order of c), and the result is (s0 + s1) + (s2 + s3),
// so the products do not wait on one accumulator chain.  dot_rows_lds reads
// 16 bytes at a time from LDS rows (16-byte aligned); dot_rows reads one
// float at a time (rows in device memory are only 4-byte aligned on this
// path).  Both sum in the same order: the same two rows give the same float.
__device__ __forceinline__ float dot_rows(const float* a, const float* b, int d) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int c = 0;
  for (; c + 4 <= d; c += 4) {
    s0 = fmaf(a[c], b[c], s0);
    s1 = fmaf(a[c + 1], b[c + 1], s1);
    s2 = fmaf(a[c + 2], b[c + 2], s2);
    s3 = fmaf(a[c + 3], b[c + 3], s3);
  }
  if (c < d) s0 = fmaf(a[c], b[c], s0);
  if (c + 1 < d) s1 = fmaf(a[c + 1], b[c + 1], s1);
  if (c + 2 < d) s2 = fmaf(a[c + 2], b[c + 2], s2);
  return (s0 + s1) + (s2 + s3);
}

__device__ __forceinline__ float dot_rows_lds(const float* a, const float* b, int d) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int c = 0;
  for (; c + 4 <= d; c += 4) {
    const float4 x = *reinterpret_cast<const float4*>(a + c);
    const float4 y = *reinterpret_cast<const float4*>(b + c);
    s0 = fmaf(x.x, y.x, s0);
    s1 = fmaf(x.y, y.y, s1);
    s2 = fmaf(x.z, y.z, s2);
    s3 = fmaf(x.w, y.w, s3);
  }
  if (c < d) s0 = fmaf(a[c], b[c], s0);
  if (c + 1 < d) s1 = fmaf(a[c + 1], b[c + 1], s1);
  if (c + 2 < d) s2 = fmaf(a[c + 2], b[c + 2], s2);
  return (s0 + s1) + (s2 + s3);
}

// grid: (ceil(N/8) * B*H); block: 64.  Lane t: query r = t/8, key j = t%8 for
// the scores; output columns c = t%8 + 8u of query r.
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ o,
                                                     float* __restrict__ lse, int N, int d,
                                                     int ntq, float scale) {
  __shared__ __attribute__((aligned(16))) float Qs[T][DMAX], Ks[T][DMAX], Vs[T][DMAX];
  const int bh = blockIdx.x / ntq, qt = blockIdx.x - bh * ntq;
  const int64_t base = (int64_t)bh * N * d;
  const int t = threadIdx.x, r = t >> 3, j = t & 7;
  const int q0 = qt * T;
  load_tile(Qs, q + base, q0, N, d);
  float m = -INFINITY, l = 0.0f;
  float acc[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) acc[u] = 0.0f;
  const int nkt = (N + T - 1) / T;
  TileRegs kr, vr;
  fetch_tile(kr, k + base, 0, N, d);
  fetch_tile(vr, v + base, 0, N, d);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    put_tile(Ks, kr, d);
    put_tile(Vs, vr, d);
    __syncthreads();
    if (kt + 1 < nkt) {
      fetch_tile(kr, k + base, (kt + 1) * T, N, d);
      fetch_tile(vr, v + base, (kt + 1) * T, N, d);
    }
    float s = scale * dot_rows_lds(Qs[r], Ks[j], d);
    if (kt * T + j >= N) s = -INFINITY;
    const float m_new = fmaxf(m, group8_max(s));
    const float alpha = expf(m - m_new);  // exp(-inf) = 0 on the first block
    const float p = expf(s - m_new);
    l = alpha * l + group8_sum(p);
#pragma unroll
    for (int u = 0; u < CPT; ++u) acc[u] *= alpha;
    for (int jj = 0; jj < T; ++jj) {
      const float pj = __shfl(p, r * T + jj);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = j + T * u;
        if (c < d) acc[u] = fmaf(pj, Vs[jj][c], acc[u]);
      }
    }
    m = m_new;
  }
  const int qi = q0 + r;
  if (qi < N) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = j + T * u;
      if (c < d) o[base + (int64_t)qi * d + c] = acc[u] * inv;
    }
    if (j == 0) lse[(int64_t)bh * N + qi] = m + logf(l);
  }
}

// D_i = sum_c dO_ic O_ic; one thread per row.
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(const float* __restrict__ o,
                                                          const float* __restrict__ dO,
                                                          float* __restrict__ delta,
                                                          int64_t rows, int d) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  delta[row] = dot_rows(o + row * d, dO + row * d, d);
}

// Loads per-query LSE and D for rows [q0, q0+T); rows past N get LSE = +inf
// (so P = 0) and D = 0.
__device__ __forceinline__ void load_row_stats(float* lse_s, float* d_s, const float* lse,
                                               const float* delta, int q0, int N) {
  const int t = threadIdx.x;
  if (t < T) {
    const bool ok = q0 + t < N;
    lse_s[t] = ok ? lse[q0 + t] : INFINITY;
    d_s[t] = ok ? delta[q0 + t] : 0.0f;
  }
}

// grid: (ceil(N/8) * B*H); block 64.  Workgroup owns keys [k0, k0+8).
// Lane t: key j = t/8, query i = t%8 for the scores; accumulates dK, dV of
// key j for columns c = t%8 + 8u.
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dO,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv, int N,
    int d, int nkt, float scale) {
  __shared__ __attribute__((aligned(16))) float Qs[T][DMAX], dOs[T][DMAX], Ks[T][DMAX], Vs[T][DMAX];
  __shared__ float lse_s[T], d_s[T];
  const int bh = blockIdx.x / nkt, kt = blockIdx.x - bh * nkt;
  const int64_t base = (int64_t)bh * N * d;
  const float* lse_h = lse + (int64_t)bh * N;
  const float* delta_h = delta + (int64_t)bh * N;
  const int t = threadIdx.x, j = t >> 3, i = t & 7;
  const int k0 = kt * T;
  load_tile(Ks, k + base, k0, N, d);
  load_tile(Vs, v + base, k0, N, d);
  float accK[CPT], accV[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) accK[u] = accV[u] = 0.0f;
  const int nqt = (N + T - 1) / T;
  TileRegs qr, gr;
  float st_l, st_d;   // LSE and D of query row t (threads t < T)
  auto fetch_q = [&](int q0) {
    fetch_tile(qr, q + base, q0, N, d);
    fetch_tile(gr, dO + base, q0, N, d);
    const bool ok = t < T && q0 + t < N;
    st_l = ok ? lse_h[q0 + t] : INFINITY;
    st_d = ok ? delta_h[q0 + t] : 0.0f;
  };
  fetch_q(0);
  for (int qt = 0; qt < nqt; ++qt) {
    __syncthreads();
    put_tile(Qs, qr, d);
    put_tile(dOs, gr, d);
    if (t < T) {
      lse_s[t] = st_l;
      d_s[t] = st_d;
    }
    __syncthreads();
    if (qt + 1 < nqt) fetch_q((qt + 1) * T);
    const float s = scale * dot_rows_lds(Qs[i], Ks[j], d);
    const float p = expf(s - lse_s[i]);
    const float dp = dot_rows_lds(dOs[i], Vs[j], d);
    const float ds = p * (dp - d_s[i]);
    for (int ii = 0; ii < T; ++ii) {
      const float pi = __shfl(p, j * T + ii);
      const float dsi = __shfl(ds, j * T + ii);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = i + T * u;
        if (c < d) {
          accV[u] = fmaf(pi, dOs[ii][c], accV[u]);
          accK[u] = fmaf(dsi, Qs[ii][c], accK[u]);
        }
      }
    }
  }
  const int kj = k0 + j;
  if (kj < N) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = i + T * u;
      if (c < d) {
        dk[base + (int64_t)kj * d + c] = scale * accK[u];
        dv[base + (int64_t)kj * d + c] = accV[u];
      }
    }
  }
}

// grid: (ceil(N/8) * B*H); block 64.  Workgroup owns queries [q0, q0+8).
// Lane t: query i = t/8, key j = t%8; accumulates dQ of query i for columns
// c = t%8 + 8u.
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dO,
    const float* __restrict__ delta, float* __restrict__ dq, int N, int d, int nqt,
    float scale) {
  __shared__ __attribute__((aligned(16))) float Qs[T][DMAX], dOs[T][DMAX], Ks[T][DMAX], Vs[T][DMAX];
  __shared__ float lse_s[T], d_s[T];
  const int bh = blockIdx.x / nqt, qt = blockIdx.x - bh * nqt;
  const int64_t base = (int64_t)bh * N * d;
  const int t = threadIdx.x, i = t >> 3, j = t & 7;
  const int q0 = qt * T;
  load_tile(Qs, q + base, q0, N, d);
  load_tile(dOs, dO + base, q0, N, d);
  load_row_stats(lse_s, d_s, lse + (int64_t)bh * N, delta + (int64_t)bh * N, q0, N);
  float acc[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) acc[u] = 0.0f;
  const int nkt = (N + T - 1) / T;
  TileRegs kr, vr;
  fetch_tile(kr, k + base, 0, N, d);
  fetch_tile(vr, v + base, 0, N, d);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    put_tile(Ks, kr, d);
    put_tile(Vs, vr, d);
    __syncthreads();
    if (kt + 1 < nkt) {
      fetch_tile(kr, k + base, (kt + 1) * T, N, d);
      fetch_tile(vr, v + base, (kt + 1) * T, N, d);
    }
    const float s = scale * dot_rows_lds(Qs[i], Ks[j], d);
    const float p = (kt * T + j < N) ? expf(s - lse_s[i]) : 0.0f;
    const float dp = dot_rows_lds(dOs[i], Vs[j], d);
    const float ds = p * (dp - d_s[i]);
    for (int jj = 0; jj < T; ++jj) {
      const float dsj = __shfl(ds, i * T + jj);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = j + T * u;
        if (c < d) acc[u] = fmaf(dsj, Ks[jj][c], acc[u]);
      }
    }
  }
  const int qi = q0 + i;
  if (qi < N) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = j + T * u;
      if (c < d) dq[base + (int64_t)qi * d + c] = scale * acc[u];
    }
  }
}

}  // namespace

bool f32_mfma_fits(int64_t N, int64_t d);
int launch_fwd_f32_mfma(const float* q, const float* k, const float* v, float* o, float* lse,
                        int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream);

int launch_bwd_f32_mfma(const float* q, const float* k, const float* v, const float* lse,
                        const float* dO, const float* delta, float* dq, float* dk, float* dv,
                        int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream);

// Keys per rescale step of the fp32 calls.  Up to kSmallN keys (the fable's
// 64 rows among them) and for head dims the matrix cores do not take, the
// kernels of this file step through blocks of 8 with the exact running max;
// longer sequences at d = 64 or 128 run on the fp32 matrix cores with blocks
// of 32.  Both are exact in real arithmetic; at the small sizes the
// matrix cores would not pay (a few workgroups, launch-bound either way).
constexpr int64_t kSmallN = 256;
int f32_key_block(int64_t N, int64_t d) {
  return (N > kSmallN && f32_mfma_fits(N, d)) ? 32 : T;
}

int launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream) {
  if (f32_key_block(N, d) != T)
    return launch_fwd_f32_mfma(q, k, v, o, lse, BH, N, d, scale, stream);
  const int64_t ntq = (N + T - 1) / T;
  return launch_in_chunks(BH, ntq * 64, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * d;
    hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)(ntq * nh)), dim3(64), 0, stream, q + off,
                       k + off, v + off, o + off, lse + h0 * N, (int)N, (int)d, (int)ntq, scale);
    return (int)hipGetLastError();
  });
}

int launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                   const float* lse, const float* dO, float* dq, float* dk, float* dv,
                   float* delta, int64_t BH, int64_t N, int64_t d, float scale,
                   hipStream_t stream) {
  const bool small = f32_key_block(N, d) == T;
  const int64_t nt = (N + T - 1) / T;
  // The 8-row kernels' grid of one head must fit one launch (checked before
  // the preprocess is enqueued; the matrix-core kernels check their own).
  if (small && !unit_fits(nt * 64)) return kErrGridTooLarge;
  const int64_t rows = BH * N;
  int e = launch_in_chunks((rows + 255) / 256, 256, [&](int64_t b0, int64_t nb) {
    const int64_t r0 = b0 * 256, nr = std::min(nb * 256, rows - r0);
    hipLaunchKernelGGL(bwd_pre_f32_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                       o + r0 * d, dO + r0 * d, delta + r0, nr, (int)d);
    return (int)hipGetLastError();
  });
  if (e != 0) return e;
  if (!small)
    return launch_bwd_f32_mfma(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, d, scale, stream);
  e = launch_in_chunks(BH, nt * 64, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * d, roff = h0 * N;
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel, dim3((unsigned)(nt * nh)), dim3(64), 0, stream,
                       q + off, k + off, v + off, lse + roff, dO + off, delta + roff, dk + off,
                       dv + off, (int)N, (int)d, (int)nt, scale);
    return (int)hipGetLastError();
  });
  if (e != 0) return e;
  return launch_in_chunks(BH, nt * 64, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * d, roff = h0 * N;
    hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)(nt * nh)), dim3(64), 0, stream,
                       q + off, k + off, v + off, lse + roff, dO + off, delta + roff, dq + off,
                       (int)N, (int)d, (int)nt, scale);
    return (int)hipGetLastError();
  });
}

}  // namespace fa
