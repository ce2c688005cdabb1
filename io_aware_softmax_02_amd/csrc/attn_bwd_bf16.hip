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
// dQ) is stored transposed and key/query-permuted (kperm16, tswz) so that
// the 8 values a lane needs are one 16-byte read and line up with the score
// accumulator layout that supplies the other operand.
//
// Streaming: the tiles of the loop are fetched with buffer loads (reads past
// the end of a head return 0, which is what a ragged last tile needs) into
// registers one tile ahead, and written to the other half of a double-buffered
// LDS area after the math on the current tile; one barrier per tile.
#include "device_common.h"

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

// A tile of 64 rows x D columns is handled as 4-row x 8-column blocks; block
// b covers rows 4*(b / (D/8)) .. +3 and columns 8*(b % (D/8)) .. +7 (consecutive
// lanes along a row, so the row-major LDS writes are conflict-free).
template <int D>
__device__ __forceinline__ void load_block(u32x4 (&r)[4], rsrc_t src, int row0, int b) {
  const int r0 = (b / (D / 8)) * 4, col = (b % (D / 8)) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = buf_load16(src, (uint32_t)(((row0 + r0 + i) * D + col) * 2));
}

// Writes a loaded block row-major into an LDS tile with pitch P (if given) and
// transposed + permuted into a swizzled 64-position tile (if given).
template <int D>
__device__ __forceinline__ void store_block(const u32x4 (&r)[4], int b, uint16_t* rowmajor, int P,
                                            uint16_t* trans) {
  const int r0 = (b / (D / 8)) * 4, col = (b % (D / 8)) * 8;
  if (rowmajor) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(rowmajor + (r0 + i) * P + col) = r[i];
  }
  if (trans) {
    const int pos = (r0 & ~15) + kperm16(r0 & 15);
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
  static constexpr int P = D + 8;            // row-major tile pitch (bf16)
  static constexpr int ROW_ELEMS = BQ * P;
  static constexpr int T_ELEMS = D * 64;     // transposed tiles (tswz layout)
  // One buffer: Qs, dOs (row-major), Qt, dOt (transposed), lse2[BQ], delta[BQ]
  static constexpr int OFF_QS = 0;
  static constexpr int OFF_DOS = OFF_QS + ROW_ELEMS;
  static constexpr int OFF_QT = OFF_DOS + ROW_ELEMS;
  static constexpr int OFF_DOT = OFF_QT + T_ELEMS;
  static constexpr int OFF_STATS = OFF_DOT + T_ELEMS;   // bf16 units; 2*BQ floats follow
  static constexpr int BUF_ELEMS = OFF_STATS + 4 * BQ;
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int NBLK = (BQ / 4) * (D / 8);         // blocks per matrix per tile
  static constexpr int BLK_PER_T = 2 * NBLK / THREADS;   // Q and dO blocks per thread
  static constexpr int DK = D / 16, DB = D / 32;
  static_assert(BQ == 64, "transposed tiles hold 64 positions per row");
  static_assert((2 * NBLK) % THREADS == 0, "whole blocks per thread");
};

template <int D>
struct DkdvTile {
  u32x4 blk[DkdvCfg<D>::BLK_PER_T][4];
  float stat;
};

template <int D>
__device__ __forceinline__ void dkdv_load(DkdvTile<D>& t, rsrc_t rq, rsrc_t rdo, rsrc_t rlse,
                                          rsrc_t rdel, int q0, int tid) {
  using C = DkdvCfg<D>;
#pragma unroll
  for (int u = 0; u < C::BLK_PER_T; ++u) {
    const int b = tid + u * C::THREADS;
    const bool isq = b < C::NBLK;
    load_block<D>(t.blk[u], isq ? rq : rdo, q0, isq ? b : b - C::NBLK);
  }
  t.stat = 0.0f;
  if (tid < 2 * C::BQ) t.stat = buf_loadf(tid < C::BQ ? rlse : rdel,
                                         (uint32_t)((q0 + (tid & (C::BQ - 1))) * 4));
}

template <int D>
__device__ __forceinline__ void dkdv_store(const DkdvTile<D>& t, uint16_t* buf, int q0, int N,
                                           int tid) {
  using C = DkdvCfg<D>;
#pragma unroll
  for (int u = 0; u < C::BLK_PER_T; ++u) {
    const int b = tid + u * C::THREADS;
    const bool isq = b < C::NBLK;
    store_block<D>(t.blk[u], isq ? b : b - C::NBLK, buf + (isq ? C::OFF_QS : C::OFF_DOS), C::P,
                   buf + (isq ? C::OFF_QT : C::OFF_DOT));
  }
  float* st = reinterpret_cast<float*>(buf + C::OFF_STATS);
  if (tid < C::BQ) {
    // log2-domain LSE; +inf past N makes P exactly 0 for rows that do not exist
    st[tid] = q0 + tid < N ? t.stat * kLog2e : INFINITY;
  } else if (tid < 2 * C::BQ) {
    st[tid] = t.stat;    // delta, 0 past N
  }
}

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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  DkdvTile<D> tile;
  dkdv_load<D>(tile, rq, rdo, rlse, rdel, 0, tid);
  dkdv_store<D>(tile, smem, 0, N, tid);
  __syncthreads();

  for (int it = 0; it < nqt; ++it) {
    const uint16_t* buf = smem + (it & 1) * C::BUF_ELEMS;
    const uint16_t* Qs = buf + C::OFF_QS;
    const uint16_t* dOs = buf + C::OFF_DOS;
    const uint16_t* Qt = buf + C::OFF_QT;
    const uint16_t* dOt = buf + C::OFF_DOT;
    const float* lse2s = reinterpret_cast<const float*>(buf + C::OFF_STATS);
    const float* dls = lse2s + C::BQ;
    const bool more = it + 1 < nqt;
    if (more) dkdv_load<D>(tile, rq, rdo, rlse, rdel, (it + 1) * C::BQ, tid);

    // S = Q K^T and dP = dO V^T for the two 32-query blocks: four
    // independent accumulator chains, with the LDS operands of k-step kk+RA
    // read before the instructions of step kk (see kReadAhead).
    f32x16 s[2], dp[2];
    {
      constexpr int RA = kReadAhead;
      const uint16_t* qrow = Qs + li * C::P + g * 8;
      const uint16_t* orow = dOs + li * C::P + g * 8;
      bf16x8 qa[RA + 1][2], oa[RA + 1][2];
#pragma unroll
      for (int kk = 0; kk < RA; ++kk)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          qa[kk][qb] = lds_bf16x8(qrow + qb * 32 * C::P + kk * 16);
          oa[kk][qb] = lds_bf16x8(orow + qb * 32 * C::P + kk * 16);
        }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[qb] = dp[qb] = zero16();
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        if (kk + RA < C::DK) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            qa[(kk + RA) % (RA + 1)][qb] = lds_bf16x8(qrow + qb * 32 * C::P + (kk + RA) * 16);
            oa[(kk + RA) % (RA + 1)][qb] = lds_bf16x8(orow + qb * 32 * C::P + (kk + RA) * 16);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb] = mfma32(qa[kk % (RA + 1)][qb], kreg[kk], s[qb]);
          dp[qb] = mfma32(oa[kk % (RA + 1)][qb], vreg[kk], dp[qb]);
        }
      }
    }
    // P and dS; element i of block qb is query qb*32 + 8*(i/4) + 4g + i%4.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qo = qb * 32 + 8 * r + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dls + qo);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(fmaf(s[qb][4 * r + e], c2, -l4[e]));
          s[qb][4 * r + e] = p;
          dp[qb][4 * r + e] = p * (dp[qb][4 * r + e] - d4[e]);
        }
      }
    // P and dS to bf16 B operands, one per 16-query step t.
    bf16x8 pb[C::BQ / 16], sb[C::BQ / 16];
#pragma unroll
    for (int t = 0; t < C::BQ / 16; ++t) {
      const int qb = t >> 1, h = t & 1;
      u32x4 pw, sw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = pack_bf16x2(s[qb][8 * h + 2 * e], s[qb][8 * h + 2 * e + 1]);
        sw[e] = pack_bf16x2(dp[qb][8 * h + 2 * e], dp[qb][8 * h + 2 * e + 1]);
      }
      pb[t] = as_bf16x8(pw);
      sb[t] = as_bf16x8(sw);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over steps n = (t, cb), operands
    // read kStepAhead steps ahead.
    {
      constexpr int RA = kStepAhead, NS = (C::BQ / 16) * C::DB;
      bf16x8 oa[RA + 1], qa[RA + 1];
#pragma unroll
      for (int n = 0; n < RA; ++n) {
        const int off = tswz((n % C::DB) * 32 + li, (n / C::DB) * 16 + g * 8);
        oa[n] = lds_bf16x8(dOt + off);
        qa[n] = lds_bf16x8(Qt + off);
      }
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + RA < NS) {
          const int m = n + RA;
          const int off = tswz((m % C::DB) * 32 + li, (m / C::DB) * 16 + g * 8);
          oa[m % (RA + 1)] = lds_bf16x8(dOt + off);
          qa[m % (RA + 1)] = lds_bf16x8(Qt + off);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int t = n / C::DB, cb = n % C::DB;
        dvt[cb] = mfma32(oa[n % (RA + 1)], pb[t], dvt[cb]);
        dkt[cb] = mfma32(qa[n % (RA + 1)], sb[t], dkt[cb]);
      }
    }

    if (more) dkdv_store<D>(tile, smem + ((it + 1) & 1) * C::BUF_ELEMS, (it + 1) * C::BQ, N, tid);
    __syncthreads();
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
  static constexpr int BQ = 128, BK = 64, THREADS = 256;
  static constexpr int P = D + 8;
  static constexpr int ROW_ELEMS = BK * P;
  static constexpr int T_ELEMS = D * 64;     // transposed tile (tswz layout)
  static constexpr int OFF_KS = 0;
  static constexpr int OFF_VS = OFF_KS + ROW_ELEMS;
  static constexpr int OFF_KT = OFF_VS + ROW_ELEMS;
  static constexpr int BUF_ELEMS = OFF_KT + T_ELEMS;
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int NBLK = (BK / 4) * (D / 8);
  static constexpr int BLK_PER_T = 2 * NBLK / THREADS;   // K and V blocks per thread
  static constexpr int DK = D / 16, DB = D / 32;
  static_assert(BK == 64, "transposed tiles hold 64 positions per row");
  static_assert((2 * NBLK) % THREADS == 0, "whole blocks per thread");
};

template <int D>
struct DqTile {
  u32x4 blk[DqCfg<D>::BLK_PER_T][4];
};

template <int D>
__device__ __forceinline__ void dq_load(DqTile<D>& t, rsrc_t rk, rsrc_t rv, int k0, int tid) {
  using C = DqCfg<D>;
#pragma unroll
  for (int u = 0; u < C::BLK_PER_T; ++u) {
    const int b = tid + u * C::THREADS;
    const bool isk = b < C::NBLK;
    load_block<D>(t.blk[u], isk ? rk : rv, k0, isk ? b : b - C::NBLK);
  }
}

template <int D>
__device__ __forceinline__ void dq_store(const DqTile<D>& t, uint16_t* buf, int tid) {
  using C = DqCfg<D>;
#pragma unroll
  for (int u = 0; u < C::BLK_PER_T; ++u) {
    const int b = tid + u * C::THREADS;
    if (b < C::NBLK)
      store_block<D>(t.blk[u], b, buf + C::OFF_KS, C::P, buf + C::OFF_KT);
    else
      store_block<D>(t.blk[u], b - C::NBLK, buf + C::OFF_VS, C::P, nullptr);
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  DqTile<D> tile;
  dq_load<D>(tile, rk, rv, 0, tid);
  dq_store<D>(tile, smem, tid);
  __syncthreads();

  for (int it = 0; it < nkt; ++it) {
    const uint16_t* buf = smem + (it & 1) * C::BUF_ELEMS;
    const uint16_t* Ks = buf + C::OFF_KS;
    const uint16_t* Vs = buf + C::OFF_VS;
    const uint16_t* Kt = buf + C::OFF_KT;
    const bool more = it + 1 < nkt;
    if (more) dq_load<D>(tile, rk, rv, (it + 1) * C::BK, tid);

    // S^T = K Q^T and dP^T = V dO^T for the two 32-key blocks, operands
    // read kReadAhead k-steps ahead.
    f32x16 s[2], dp[2];
    {
      constexpr int RA = kReadAhead;
      const uint16_t* krow = Ks + li * C::P + g * 8;
      const uint16_t* vrow = Vs + li * C::P + g * 8;
      bf16x8 ka[RA + 1][2], va[RA + 1][2];
#pragma unroll
      for (int kk = 0; kk < RA; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          ka[kk][kb] = lds_bf16x8(krow + kb * 32 * C::P + kk * 16);
          va[kk][kb] = lds_bf16x8(vrow + kb * 32 * C::P + kk * 16);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = dp[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        if (kk + RA < C::DK) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            ka[(kk + RA) % (RA + 1)][kb] = lds_bf16x8(krow + kb * 32 * C::P + (kk + RA) * 16);
            va[(kk + RA) % (RA + 1)][kb] = lds_bf16x8(vrow + kb * 32 * C::P + (kk + RA) * 16);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = mfma32(ka[kk % (RA + 1)][kb], qreg[kk], s[kb]);
          dp[kb] = mfma32(va[kk % (RA + 1)][kb], oreg[kk], dp[kb]);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[kb][i], c2, -lse2));
        dp[kb][i] = p * (dp[kb][i] - dl);
      }
    bf16x8 sb[C::BK / 16];
#pragma unroll
    for (int t = 0; t < C::BK / 16; ++t) {
      const int kb = t >> 1, h = t & 1;
      u32x4 sw;
#pragma unroll
      for (int e = 0; e < 4; ++e) sw[e] = pack_bf16x2(dp[kb][8 * h + 2 * e], dp[kb][8 * h + 2 * e + 1]);
      sb[t] = as_bf16x8(sw);
    }
    // dQ^T += K^T dS^T over steps n = (t, cb), operands read kStepAhead
    // steps ahead.
    {
      constexpr int RA = kStepAhead, NS = (C::BK / 16) * C::DB;
      bf16x8 ka[RA + 1];
#pragma unroll
      for (int n = 0; n < RA; ++n)
        ka[n] = lds_bf16x8(Kt + tswz((n % C::DB) * 32 + li, (n / C::DB) * 16 + g * 8));
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + RA < NS) {
          const int m = n + RA;
          ka[m % (RA + 1)] = lds_bf16x8(Kt + tswz((m % C::DB) * 32 + li, (m / C::DB) * 16 + g * 8));
        }
        __builtin_amdgcn_sched_barrier(0);
        const int cb = n % C::DB;
        dqt[cb] = mfma32(ka[n % (RA + 1)], sb[n / C::DB], dqt[cb]);
      }
    }

    if (more) dq_store<D>(tile, smem + ((it + 1) & 1) * C::BUF_ELEMS, tid);
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
