// bf16 attention backward for gfx950 with recomputation: P is rebuilt from
// Q, K and the forward's per-row LSE instead of being stored (账房先生的奔命,
// carrie-l.github.io, section 七).  The gradients are the chain rule through
// O = softmax(s Q K^T) V:
//   D  = rowsum(dO * O)               (preprocess kernel)
//   P  = exp(s Q K^T - LSE)           (recomputed per tile)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK = s dS^T Q                     (dK/dV kernel, keys resident)
//   dQ = s dS K                       (dQ kernel, queries resident)
// The dQ pass is separate (it recomputes S, P and dP for its own tiles), so
// every output is written once, in a fixed order, without atomics.
//
// Matrix-core layout as in device_common.h.  Each contraction keeps one
// operand in registers and reads the other from LDS; an operand whose
// contraction index runs along a tile's rows (Q^T in dK, dO^T in dV, K^T in
// dQ) is stored transposed and key/query-permuted (kperm16) so that the
// 8 values a lane needs are one 16-byte read and line up with the score
// accumulator layout that supplies the other operand.
#include "device_common.h"

namespace fa {
namespace {

__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int x = wg & 7, idx = wg >> 3;
  const int base = nwg >> 3, rem = nwg & 7;
  return x * base + (x < rem ? x : rem) + idx;
}

// ---------------------------------------------------------------------------
// Preprocess: D_i = sum_c dO_ic O_ic (fp32).  D/8 lanes per row, 16 B each.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta, int64_t rows) {
  constexpr int LPR = D / 8;                    // lanes per row
  constexpr int RPB = 256 / LPR;                // rows per block
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int col = (tid % LPR) * 8;
  float s = 0.0f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + col);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + col);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), s);
      s = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), s);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && tid % LPR == 0) delta[row] = s;
}

// Loads a 4-row x 8-column block of a [N][D] bf16 matrix (rows >= N are 0).
template <int D>
__device__ __forceinline__ void load_block4x8(u32x4 (&r)[4], const uint16_t* __restrict__ src,
                                              int row0, int col, int N) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row0 + i < N) val = *reinterpret_cast<const u32x4*>(src + (int64_t)(row0 + i) * D + col);
    r[i] = val;
  }
}

// Writes a loaded 4x8 block row-major into an LDS tile with pitch P, and
// transposed + permuted into a swizzled 64-position tile (tswz; row = column
// of the source; within each 16-row step the source rows are placed by
// kperm16).
__device__ __forceinline__ void store_block4x8(const u32x4 (&r)[4], uint16_t* rowmajor, int P,
                                               uint16_t* trans, int row0, int col) {
  if (rowmajor) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(rowmajor + (row0 + i) * P + col) = r[i];
  }
  const int pos = (row0 & ~15) + kperm16(row0 & 15);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint32_t lo, hi;
    if (c & 1) {
      lo = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
      hi = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
    } else {
      lo = (r[0][w] & 0xffffu) | (r[1][w] << 16);
      hi = (r[2][w] & 0xffffu) | (r[3][w] << 16);
    }
    u32x2 pr = {lo, hi};
    *reinterpret_cast<u32x2*>(trans + tswz(col + c, pos)) = pr;
  }
}

// ---------------------------------------------------------------------------
// dK / dV: workgroup owns 128 keys (4 waves x 32), loops over 64-query tiles.
// Per wave and tile (lane l: key l%32 of the wave's block, k-group g):
//   S  = Q K^T     (rows = queries, cols = keys; A = Q rows from LDS, B = K regs)
//   dP = dO V^T    (A = dO rows from LDS, B = V regs)
//   P  = 2^(c S - LSE log2 e), dS = P (dP - D)        (per-element, fp32)
//   dV^T += dO^T P (A = dO^T from LDS, B = P from the S accumulators)
//   dK^T += Q^T dS (A = Q^T from LDS,  B = dS)
// ---------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
  static constexpr int BK = 128, BQ = 64, THREADS = 256;
  static constexpr int P = D + 8;        // row-major tile pitch (bf16)
  static constexpr int ROW_ELEMS = BQ * P;
  static constexpr int T_ELEMS = D * 64;  // transposed tiles (tswz layout)
  // LDS: Qs, dOs (row-major), Qt, dOt (transposed), lse2[BQ], delta[BQ]
  static constexpr int OFF_QS = 0;
  static constexpr int OFF_DOS = OFF_QS + ROW_ELEMS;
  static constexpr int OFF_QT = OFF_DOS + ROW_ELEMS;
  static constexpr int OFF_DOT = OFF_QT + T_ELEMS;
  static constexpr int OFF_STATS = OFF_DOT + T_ELEMS;  // in bf16 units; floats follow
  static constexpr int LDS_BYTES = OFF_STATS * 2 + 2 * BQ * 4;
  static constexpr int NBLK = (BQ / 4) * (D / 8);       // 4x8 blocks per tile matrix
  static constexpr int DK = D / 16, DB = D / 32;
  static_assert(BQ == 64, "transposed tiles hold 64 positions per row");
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int nkt, float c2,
    float scale) {
  using C = DkdvCfg<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* Qs = smem + C::OFF_QS;
  uint16_t* dOs = smem + C::OFF_DOS;
  uint16_t* Qt = smem + C::OFF_QT;
  uint16_t* dOt = smem + C::OFF_DOT;
  float* lse2s = reinterpret_cast<float*>(smem + C::OFF_STATS);
  float* ds_ = lse2s + C::BQ;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nkt, kt = logical - bh * nkt;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint16_t* qh = q + hoff;
  const uint16_t* doh = dO + hoff;
  const float* lseh = lse + (int64_t)bh * N;
  const float* delh = delta + (int64_t)bh * N;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, g = lane >> 5;
  const int key = kt * C::BK + wave * 32 + li;   // this lane's key row

  // K and V rows of this lane's key as B operands (k-step kk: cols kk*16+8g..).
  bf16x8 kreg[C::DK], vreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < N) {
      a = *reinterpret_cast<const u32x4*>(k + hoff + (int64_t)key * D + kk * 16 + g * 8);
      b = *reinterpret_cast<const u32x4*>(v + hoff + (int64_t)key * D + kk * 16 + g * 8);
    }
    kreg[kk] = as_bf16x8(a);
    vreg[kk] = as_bf16x8(b);
  }
  f32x16 dvt[C::DB], dkt[C::DB];
#pragma unroll
  for (int cb = 0; cb < C::DB; ++cb) dvt[cb] = dkt[cb] = zero16();

  const int nqt = (N + C::BQ - 1) / C::BQ;
  for (int it = 0; it < nqt; ++it) {
    const int q0 = it * C::BQ;
    __syncthreads();   // previous tile fully consumed
    for (int b = tid; b < 2 * C::NBLK; b += C::THREADS) {
      const bool isq = b < C::NBLK;
      const int bb = isq ? b : b - C::NBLK;
      const int r0 = (bb / (D / 8)) * 4, col = (bb % (D / 8)) * 8;
      u32x4 r[4];
      load_block4x8<D>(r, (isq ? qh : doh), q0 + r0, col, N);
      store_block4x8(r, isq ? Qs : dOs, C::P, isq ? Qt : dOt, r0, col);
    }
    if (tid < C::BQ) {
      const int qi = q0 + tid;
      lse2s[tid] = qi < N ? lseh[qi] * kLog2e : INFINITY;   // P = 0 past N
      ds_[tid] = qi < N ? delh[qi] : 0.0f;
    }
    __syncthreads();

    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = zero16();
      dp[qb] = zero16();
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        const int off = (qb * 32 + li) * C::P + kk * 16 + g * 8;
        s[qb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(Qs + off)), kreg[kk], s[qb]);
        dp[qb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(dOs + off)), vreg[kk], dp[qb]);
      }
    }
    // P and dS; element i of block qb is query qb*32 + 8*(i/4) + 4g + i%4.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qo = qb * 32 + 8 * r + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(ds_ + qo);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(fmaf(s[qb][4 * r + e], c2, -l4[e]));
          s[qb][4 * r + e] = p;
          dp[qb][4 * r + e] = p * (dp[qb][4 * r + e] - d4[e]);
        }
      }
#pragma unroll
    for (int t = 0; t < C::BQ / 16; ++t) {
      const int qb = t >> 1, h = t & 1;
      u32x4 pw, sw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = pack_bf16x2(s[qb][8 * h + 2 * e], s[qb][8 * h + 2 * e + 1]);
        sw[e] = pack_bf16x2(dp[qb][8 * h + 2 * e], dp[qb][8 * h + 2 * e + 1]);
      }
      const bf16x8 pb = as_bf16x8(pw), sb = as_bf16x8(sw);
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
        const int off = tswz(cb * 32 + li, t * 16 + g * 8);
        dvt[cb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(dOt + off)), pb, dvt[cb]);
        dkt[cb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(Qt + off)), sb, dkt[cb]);
      }
    }
  }

  // dV^T / dK^T element i of block cb: column cb*32 + 8*(i/4) + 4g + i%4 of
  // this lane's key row.
  if (key < N) {
    uint16_t* dkr = dk + hoff + (int64_t)key * D;
    uint16_t* dvr = dv + hoff + (int64_t)key * D;
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = cb * 32 + 8 * r + 4 * g;
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dkt[cb][4 * r] * scale, dkt[cb][4 * r + 1] * scale);
        wk[1] = pack_bf16x2(dkt[cb][4 * r + 2] * scale, dkt[cb][4 * r + 3] * scale);
        wv[0] = pack_bf16x2(dvt[cb][4 * r], dvt[cb][4 * r + 1]);
        wv[1] = pack_bf16x2(dvt[cb][4 * r + 2], dvt[cb][4 * r + 3]);
        *reinterpret_cast<u32x2*>(dkr + col) = wk;
        *reinterpret_cast<u32x2*>(dvr + col) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup owns 128 queries (4 waves x 32), loops over 64-key tiles.
// Per wave and tile (lane l: query l%32 of the wave's block):
//   S^T  = K Q^T    (A = K rows from LDS, B = Q regs)
//   dP^T = V dO^T   (A = V rows from LDS, B = dO regs)
//   P^T = 2^(c S^T - LSE log2 e), dS^T = P^T (dP^T - D)   (lane-uniform stats)
//   dQ^T += K^T dS^T (A = K^T from LDS, B = dS^T from the accumulators)
// ---------------------------------------------------------------------------
template <int D>
struct DqCfg {
  static constexpr int BQ = 128, BK = 64, THREADS = 256;
  static constexpr int P = D + 8;
  static constexpr int ROW_ELEMS = BK * P;
  static constexpr int T_ELEMS = D * 64;  // transposed tile (tswz layout)
  static constexpr int OFF_KS = 0;
  static constexpr int OFF_VS = OFF_KS + ROW_ELEMS;
  static constexpr int OFF_KT = OFF_VS + ROW_ELEMS;
  static constexpr int LDS_BYTES = (OFF_KT + T_ELEMS) * 2;
  static constexpr int NBLK = (BK / 4) * (D / 8);
  static constexpr int DK = D / 16, DB = D / 32;
  static_assert(BK == 64, "transposed tiles hold 64 positions per row");
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int N, int nqt, float c2, float scale) {
  using C = DqCfg<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* Ks = smem + C::OFF_KS;
  uint16_t* Vs = smem + C::OFF_VS;
  uint16_t* Kt = smem + C::OFF_KT;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint16_t* kh = k + hoff;
  const uint16_t* vh = v + hoff;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, g = lane >> 5;
  const int qrow = qt * C::BQ + wave * 32 + li;

  bf16x8 qreg[C::DK], oreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      a = *reinterpret_cast<const u32x4*>(q + hoff + (int64_t)qrow * D + kk * 16 + g * 8);
      b = *reinterpret_cast<const u32x4*>(dO + hoff + (int64_t)qrow * D + kk * 16 + g * 8);
    }
    qreg[kk] = as_bf16x8(a);
    oreg[kk] = as_bf16x8(b);
  }
  const float lse2 = qrow < N ? lse[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dl = qrow < N ? delta[(int64_t)bh * N + qrow] : 0.0f;

  f32x16 dqt[C::DB];
#pragma unroll
  for (int cb = 0; cb < C::DB; ++cb) dqt[cb] = zero16();

  const int nkt = (N + C::BK - 1) / C::BK;
  for (int it = 0; it < nkt; ++it) {
    const int k0 = it * C::BK;
    __syncthreads();
    for (int b = tid; b < 2 * C::NBLK; b += C::THREADS) {
      const bool isk = b < C::NBLK;
      const int bb = isk ? b : b - C::NBLK;
      const int r0 = (bb / (D / 8)) * 4, col = (bb % (D / 8)) * 8;
      u32x4 r[4];
      load_block4x8<D>(r, isk ? kh : vh, k0 + r0, col, N);
      if (isk) {
        store_block4x8(r, Ks, C::P, Kt, r0, col);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(Vs + (r0 + i) * C::P + col) = r[i];
      }
    }
    __syncthreads();

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
      dp[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        const int off = (kb * 32 + li) * C::P + kk * 16 + g * 8;
        s[kb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + off)), qreg[kk], s[kb]);
        dp[kb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(Vs + off)), oreg[kk], dp[kb]);
      }
    }
    // Keys past N are zero rows of K and V, so their dS multiplies a zero
    // row of K^T below and adds nothing to dQ.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[kb][i], c2, -lse2));
        dp[kb][i] = p * (dp[kb][i] - dl);
      }
#pragma unroll
    for (int t = 0; t < C::BK / 16; ++t) {
      const int kb = t >> 1, h = t & 1;
      u32x4 sw;
#pragma unroll
      for (int e = 0; e < 4; ++e) sw[e] = pack_bf16x2(dp[kb][8 * h + 2 * e], dp[kb][8 * h + 2 * e + 1]);
      const bf16x8 sb = as_bf16x8(sw);
#pragma unroll
      for (int cb = 0; cb < C::DB; ++cb) {
        const int off = tswz(cb * 32 + li, t * 16 + g * 8);
        dqt[cb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(Kt + off)), sb, dqt[cb]);
      }
    }
  }

  if (qrow < N) {
    uint16_t* dqr = dq + hoff + (int64_t)qrow * D;
#pragma unroll
    for (int cb = 0; cb < C::DB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(dqt[cb][4 * r] * scale, dqt[cb][4 * r + 1] * scale);
        w[1] = pack_bf16x2(dqt[cb][4 * r + 2] * scale, dqt[cb][4 * r + 3] * scale);
        *reinterpret_cast<u32x2*>(dqr + cb * 32 + 8 * r + 4 * g) = w;
      }
  }
}

template <typename F>
hipError_t allow_lds(F* kernel, int bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             bytes);
}

template <int D>
int launch_pre(const uint16_t* o, const uint16_t* dO, float* delta, int64_t rows,
               hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, o, dO, delta, rows);
  return (int)hipGetLastError();
}

template <int D>
int launch_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                const uint16_t* dO, const float* delta, uint16_t* dk, uint16_t* dv, int64_t BH,
                int64_t N, float scale, hipStream_t stream) {
  using C = DkdvCfg<D>;
  hipError_t e = allow_lds(bwd_dkdv_kernel<D>, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  const int nkt = (int)((N + C::BK - 1) / C::BK);
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(nkt * BH)), dim3(C::THREADS),
                     C::LDS_BYTES, stream, q, k, v, lse, dO, delta, dk, dv, (int)N, nkt,
                     scale * kLog2e, scale);
  return (int)hipGetLastError();
}

template <int D>
int launch_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
              const uint16_t* dO, const float* delta, uint16_t* dq, int64_t BH, int64_t N,
              float scale, hipStream_t stream) {
  using C = DqCfg<D>;
  hipError_t e = allow_lds(bwd_dq_kernel<D>, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  const int nqt = (int)((N + C::BQ - 1) / C::BQ);
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(nqt * BH)), dim3(C::THREADS),
                     C::LDS_BYTES, stream, q, k, v, lse, dO, delta, dq, (int)N, nqt,
                     scale * kLog2e, scale);
  return (int)hipGetLastError();
}

}  // namespace

int launch_bwd_pre_bf16(const void* o, const void* dO, float* delta, int64_t rows, int64_t d,
                        hipStream_t stream) {
  const auto* o16 = static_cast<const uint16_t*>(o);
  const auto* g16 = static_cast<const uint16_t*>(dO);
  return d == 128 ? launch_pre<128>(o16, g16, delta, rows, stream)
                  : launch_pre<64>(o16, g16, delta, rows, stream);
}

int launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const float* lse,
                         const void* dO, const float* delta, void* dk, void* dv, int64_t BH,
                         int64_t N, int64_t d, float scale, hipStream_t stream) {
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* g16 = static_cast<const uint16_t*>(dO);
  auto* dk16 = static_cast<uint16_t*>(dk);
  auto* dv16 = static_cast<uint16_t*>(dv);
  return d == 128
             ? launch_dkdv<128>(q16, k16, v16, lse, g16, delta, dk16, dv16, BH, N, scale, stream)
             : launch_dkdv<64>(q16, k16, v16, lse, g16, delta, dk16, dv16, BH, N, scale, stream);
}

int launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const float* lse,
                       const void* dO, const float* delta, void* dq, int64_t BH, int64_t N,
                       int64_t d, float scale, hipStream_t stream) {
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* g16 = static_cast<const uint16_t*>(dO);
  auto* dq16 = static_cast<uint16_t*>(dq);
  return d == 128 ? launch_dq<128>(q16, k16, v16, lse, g16, delta, dq16, BH, N, scale, stream)
                  : launch_dq<64>(q16, k16, v16, lse, g16, delta, dq16, BH, N, scale, stream);
}

}  // namespace fa
