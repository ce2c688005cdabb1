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
// operand in registers and reads the other from a row-major LDS tile
// (lds_tile.h): along rows for S, dP and their transposes, and with
// transposing reads for the operands whose contraction index runs along the
// tile's rows (Q^T in dK, dO^T in dV, K^T in dQ), in the key/query order of
// the score accumulators that supply the other operand.
//
// Streaming: the tiles of the loop are fetched one tile ahead with direct
// buffer->LDS loads (reads past the end of a head return 0, which is what a
// ragged last tile needs) into the other half of a double-buffered LDS
// area; one barrier per tile.
#include "lds_tile.h"

namespace fa {
namespace {

// LDS operands are read this many k-steps (S, dP) or (t, cb) steps (dV,
// dK, dQ) ahead of the matrix-core instructions that use them; a scheduling
// fence between the reads and the instructions keeps the compiler from
// sinking each read next to its use, which would expose the LDS latency once
// per instruction.
constexpr int kReadAhead = 2;
constexpr int kStepAhead = 4;

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
  static constexpr int BK = 128, BQ = 64, WAVES = 4, THREADS = 64 * WAVES;
  static constexpr int TILE = BQ * D;          // one Q or dO tile (bf16), swizzled
  // One buffer: Q tile, dO tile, lse2[BQ], delta[BQ]
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = TILE;
  static constexpr int OFF_STATS = 2 * TILE;   // bf16 units; 2*BQ floats follow
  static constexpr int BUF_ELEMS = OFF_STATS + 4 * BQ;
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int DK = D / 16, DB = D / 32;
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

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nkt, kt = logical - bh * nkt;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint32_t hbytes = (uint32_t)N * D * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes);
  const rsrc_t rdo = make_rsrc(dO + hoff, hbytes);
  const rsrc_t rk = make_rsrc(k + hoff, hbytes);
  const rsrc_t rv = make_rsrc(v + hoff, hbytes);
  const rsrc_t rlse = make_rsrc(lse + (int64_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rdel = make_rsrc(delta + (int64_t)bh * N, (uint32_t)N * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int key = kt * C::BK + wave * 32 + li;   // this lane's key row

  // K and V rows of this lane's key as B operands (k-step kk: cols kk*16+8g..).
  bf16x8 kreg[C::DK], vreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    const uint32_t off = (uint32_t)((key * D + kk * 16 + g * 8) * 2);
    kreg[kk] = as_bf16x8(buf_load16(rk, off));
    vreg[kk] = as_bf16x8(buf_load16(rv, off));
  }
  f32x16 dvt[C::DB], dkt[C::DB];
#pragma unroll
  for (int cb = 0; cb < C::DB; ++cb) dvt[cb] = dkt[cb] = zero16();

  const int nqt = (N + C::BQ - 1) / C::BQ;
  // Per-row statistics of a query tile: threads 0..BQ-1 carry LSE (stored
  // in log2 units, +inf past N so that P is exactly 0 there), threads
  // BQ..2BQ-1 carry delta (0 past N).
  auto load_stat = [&](int q0) -> float {
    if (tid < 2 * C::BQ)
      return buf_loadf(tid < C::BQ ? rlse : rdel, (uint32_t)((q0 + (tid & (C::BQ - 1))) * 4));
    return 0.0f;
  };
  auto store_stat = [&](uint16_t* buf, int q0, float v) {
    float* st = reinterpret_cast<float*>(buf + C::OFF_STATS);
    if (tid < C::BQ)
      st[tid] = q0 + tid < N ? v * kLog2e : INFINITY;
    else if (tid < 2 * C::BQ)
      st[tid] = v;
  };
  tile_load<D, C::BQ, C::WAVES>(smem + C::OFF_Q, rq, 0, wave, lane);
  tile_load<D, C::BQ, C::WAVES>(smem + C::OFF_DO, rdo, 0, wave, lane);
  store_stat(smem, 0, load_stat(0));
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < nqt; ++it) {
    const uint16_t* buf = smem + (it & 1) * C::BUF_ELEMS;
    const uint16_t* Qs = buf + C::OFF_Q;
    const uint16_t* dOs = buf + C::OFF_DO;
    const float* lse2s = reinterpret_cast<const float*>(buf + C::OFF_STATS);
    const float* dls = lse2s + C::BQ;
    const bool more = it + 1 < nqt;
    uint16_t* nbuf = smem + ((it + 1) & 1) * C::BUF_ELEMS;
    float stat = 0.0f;
    if (more) {
      tile_load<D, C::BQ, C::WAVES>(nbuf + C::OFF_Q, rq, (it + 1) * C::BQ, wave, lane);
      tile_load<D, C::BQ, C::WAVES>(nbuf + C::OFF_DO, rdo, (it + 1) * C::BQ, wave, lane);
      stat = load_stat((it + 1) * C::BQ);
    }

    // One 32-query block at a time: S = Q K^T and dP = dO V^T (operands
    // read kReadAhead k-steps ahead), then P and dS, then dV^T += dO^T P and
    // dK^T += Q^T dS for the block's two 16-query steps (dO^T and Q^T
    // gathered with transposing reads kStepAhead steps ahead).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = zero16(), dp = zero16();
      {
        constexpr int RA = kReadAhead;
        bf16x8 qa[RA + 1], oa[RA + 1];
#pragma unroll
        for (int kk = 0; kk < RA; ++kk) {
          qa[kk] = row_operand<D>(Qs, qb * 32 + li, 2 * kk + g);
          oa[kk] = row_operand<D>(dOs, qb * 32 + li, 2 * kk + g);
        }
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
          if (kk + RA < C::DK) {
            qa[(kk + RA) % (RA + 1)] = row_operand<D>(Qs, qb * 32 + li, 2 * (kk + RA) + g);
            oa[(kk + RA) % (RA + 1)] = row_operand<D>(dOs, qb * 32 + li, 2 * (kk + RA) + g);
          }
          __builtin_amdgcn_sched_barrier(0);
          s = mfma32(qa[kk % (RA + 1)], kreg[kk], s);
          dp = mfma32(oa[kk % (RA + 1)], vreg[kk], dp);
        }
      }
      // P and dS; element 4r + e is query qb*32 + 8r + 4g + e.
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 pw, sw;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int r = 2 * h + rr;
          const int qo = qb * 32 + 8 * r + 4 * g;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qo);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dls + qo);
          float p[4], d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = fast_exp2(fmaf(s[4 * r + e], c2, -l4[e]));
            d[e] = p[e] * (dp[4 * r + e] - d4[e]);
          }
          pw[2 * rr] = pack_bf16x2(p[0], p[1]);
          pw[2 * rr + 1] = pack_bf16x2(p[2], p[3]);
          sw[2 * rr] = pack_bf16x2(d[0], d[1]);
          sw[2 * rr + 1] = pack_bf16x2(d[2], d[3]);
        }
        pb[h] = as_bf16x8(pw);
        sb[h] = as_bf16x8(sw);
      }
      {
        constexpr int SA = kStepAhead, NS = 2 * C::DB;   // steps n = (h, cb)
        bf16x8 oa[SA + 1], qa[SA + 1];
#pragma unroll
        for (int n = 0; n < SA; ++n) {
          oa[n] = tr_operand<D>(dOs, (2 * qb + n / C::DB) * 16, (n % C::DB) * 32, lane);
          qa[n] = tr_operand<D>(Qs, (2 * qb + n / C::DB) * 16, (n % C::DB) * 32, lane);
        }
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (n + SA < NS) {
            const int m = n + SA;
            oa[m % (SA + 1)] = tr_operand<D>(dOs, (2 * qb + m / C::DB) * 16, (m % C::DB) * 32, lane);
            qa[m % (SA + 1)] = tr_operand<D>(Qs, (2 * qb + m / C::DB) * 16, (m % C::DB) * 32, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
          const int h = n / C::DB, cb = n % C::DB;
          dvt[cb] = mfma32(oa[n % (SA + 1)], pb[h], dvt[cb]);
          dkt[cb] = mfma32(qa[n % (SA + 1)], sb[h], dkt[cb]);
        }
      }
    }

    if (more) store_stat(nbuf, (it + 1) * C::BQ, stat);
    wait_vmem();      // this wave's loads of the next tile have landed
    __syncthreads();  // ... and everyone's; the current tile is no longer read
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
// Keys past N read as zero rows of K and V, so their dS multiplies a zero row
// of K^T and adds nothing to dQ.
// ---------------------------------------------------------------------------
template <int D>
struct DqCfg {
  static constexpr int BQ = 128, BK = 64, WAVES = 4, THREADS = 64 * WAVES;
  static constexpr int TILE = BK * D;          // one K or V tile (bf16), swizzled
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = TILE;
  static constexpr int BUF_ELEMS = 2 * TILE;
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int DK = D / 16, DB = D / 32;
};

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int N, int nqt, float c2, float scale) {
  using C = DqCfg<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint32_t hbytes = (uint32_t)N * D * 2;
  const rsrc_t rk = make_rsrc(k + hoff, hbytes);
  const rsrc_t rv = make_rsrc(v + hoff, hbytes);
  const rsrc_t rq = make_rsrc(q + hoff, hbytes);
  const rsrc_t rdo = make_rsrc(dO + hoff, hbytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int qrow = qt * C::BQ + wave * 32 + li;

  bf16x8 qreg[C::DK], oreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    const uint32_t off = (uint32_t)((qrow * D + kk * 16 + g * 8) * 2);
    qreg[kk] = as_bf16x8(buf_load16(rq, off));
    oreg[kk] = as_bf16x8(buf_load16(rdo, off));
  }
  const float lse2 = qrow < N ? lse[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dl = qrow < N ? delta[(int64_t)bh * N + qrow] : 0.0f;

  f32x16 dqt[C::DB];
#pragma unroll
  for (int cb = 0; cb < C::DB; ++cb) dqt[cb] = zero16();

  const int nkt = (N + C::BK - 1) / C::BK;
  tile_load<D, C::BK, C::WAVES>(smem + C::OFF_K, rk, 0, wave, lane);
  tile_load<D, C::BK, C::WAVES>(smem + C::OFF_V, rv, 0, wave, lane);
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < nkt; ++it) {
    const uint16_t* buf = smem + (it & 1) * C::BUF_ELEMS;
    const uint16_t* Ks = buf + C::OFF_K;
    const uint16_t* Vs = buf + C::OFF_V;
    if (it + 1 < nkt) {
      uint16_t* nbuf = smem + ((it + 1) & 1) * C::BUF_ELEMS;
      tile_load<D, C::BK, C::WAVES>(nbuf + C::OFF_K, rk, (it + 1) * C::BK, wave, lane);
      tile_load<D, C::BK, C::WAVES>(nbuf + C::OFF_V, rv, (it + 1) * C::BK, wave, lane);
    }

    // One 32-key block at a time: S^T = K Q^T and dP^T = V dO^T (operands
    // read kReadAhead k-steps ahead), then P^T and dS^T for this lane's
    // query, then dQ^T += K^T dS^T for the block's two 16-key steps (K^T
    // gathered with transposing reads kStepAhead steps ahead).  Only one
    // block's scores are live at a time.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
      {
        constexpr int RA = kReadAhead;
        bf16x8 ka[RA + 1], va[RA + 1];
#pragma unroll
        for (int kk = 0; kk < RA; ++kk) {
          ka[kk] = row_operand<D>(Ks, kb * 32 + li, 2 * kk + g);
          va[kk] = row_operand<D>(Vs, kb * 32 + li, 2 * kk + g);
        }
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
          if (kk + RA < C::DK) {
            ka[(kk + RA) % (RA + 1)] = row_operand<D>(Ks, kb * 32 + li, 2 * (kk + RA) + g);
            va[(kk + RA) % (RA + 1)] = row_operand<D>(Vs, kb * 32 + li, 2 * (kk + RA) + g);
          }
          __builtin_amdgcn_sched_barrier(0);
          s = mfma32(ka[kk % (RA + 1)], qreg[kk], s);
          dp = mfma32(va[kk % (RA + 1)], oreg[kk], dp);
        }
      }
      bf16x8 sb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 sw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[8 * h + 2 * e], c2, -lse2));
          const float p1 = fast_exp2(fmaf(s[8 * h + 2 * e + 1], c2, -lse2));
          sw[e] = pack_bf16x2(p0 * (dp[8 * h + 2 * e] - dl), p1 * (dp[8 * h + 2 * e + 1] - dl));
        }
        sb[h] = as_bf16x8(sw);
      }
      {
        constexpr int SA = kStepAhead, NS = 2 * C::DB;   // steps n = (h, cb)
        bf16x8 ka[SA + 1];
#pragma unroll
        for (int n = 0; n < SA; ++n)
          ka[n] = tr_operand<D>(Ks, (2 * kb + n / C::DB) * 16, (n % C::DB) * 32, lane);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (n + SA < NS) {
            const int m = n + SA;
            ka[m % (SA + 1)] = tr_operand<D>(Ks, (2 * kb + m / C::DB) * 16, (m % C::DB) * 32, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
          const int cb = n % C::DB;
          dqt[cb] = mfma32(ka[n % (SA + 1)], sb[n / C::DB], dqt[cb]);
        }
      }
    }

    wait_vmem();
    __syncthreads();
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
