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
// Matrix-core layout as in device_common.h (dK/dV on the 32 x 32 x 16 form,
// dQ on the 16 x 16 x 32 form).  Each contraction keeps one operand in
// registers and reads the other from an LDS tile (lds_tile.h): along rows
// for S, dP and their transposes, and with transposing reads for the
// operands whose contraction index runs along the tile's rows (Q^T in dK,
// dO^T in dV, K^T in dQ), in the key/query order of the score accumulators
// that supply the other operand.  dK/dV uses row-major swizzled tiles, dQ
// row-segment tiles.
//
// Streaming: the tiles of the loop are fetched ahead with direct
// buffer->LDS loads (reads past the end of a head return 0, which is what a
// ragged last tile needs): dQ double-buffers its K/V tiles with one barrier
// per tile; dK/dV triple-buffers its Q/dO tiles (below).
#include <type_traits>

#include "launch_chunks.h"
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
constexpr int kDkdvStepAhead = 4;
constexpr int kDkdvReadAhead = 2;

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
// Per wave and 32-query block j (lane l: key l%32 of the wave's block, k-group g):
//   A(j): S  = Q K^T  (rows = queries, cols = keys; A = Q rows from LDS, B = K regs)
//         dP = dO V^T (A = dO rows from LDS, B = V regs)
//   B(j): P  = 2^(c S'), dS = P dP'                          (per-element, fp32)
// where S' = S - LSE/s and dP' = dP - D come out of the contractions directly
// (c = s log2 e): each contraction has one more k-step whose A operand holds
// -LSE/s (resp. -D) of the lane's query row split exactly into three bf16
// parts (8 + 8 + 8 significand bits) and whose B operand is (1, 1, 1, 0, ..).
// That step is issued last, so its operand is built while the others run.
// Query rows past N read as zero rows of Q and dO with LSE = D = 0, so their
// P is 1 but multiplies a zero row of dO, and their dS is 0.
//   C(j): dV^T += dO^T P (A = dO^T from LDS, B = P from the S accumulators)
//         dK^T += Q^T dS (A = Q^T from LDS,  B = dS)
// Software pipeline: the vector work B(j) runs between the matrix-core
// instructions of C(j-1) (P and dS of two blocks alternate), so the order is
// A(j), B(j) | C(j-1), A(j+1), B(j+1) | C(j), ...  B itself is split in two
// stages (scale + exp, then multiply + pack) that are one C step apart, so
// that no vector instruction between two matrix-core instructions waits on
// another.  K and V stay in accumulation registers, which the matrix cores
// read directly.
// Tiles are triple-buffered with one barrier per tile, three C steps before
// the first A of the tile it publishes (the A's first operands are read
// right after it); the loads of the tile after next are issued one
// instruction at a time between the matrix-core instructions of the A phases,
// into the buffer whose last reader (a C phase) finished before the barrier.
// Loads past the last tile read as zeros and only feed A and B work that no
// C consumes.
// ---------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
  static constexpr int BK = 128, BQ = 64, WAVES = 4, THREADS = 64 * WAVES, NBUF = 3;
  static constexpr int TILE = BQ * D;          // one 64-row tile of Q or dO (bf16), swizzled
  // One buffer: Q tile, dO tile, LSE [BQ], delta [BQ] (fp32), and a spare
  // copy of both (waves 2 and 3 load it so that no wave branches).
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = TILE;
  static constexpr int OFF_STATS = 2 * TILE;   // bf16 units; 2*BQ floats follow
  static constexpr int BUF_ELEMS = OFF_STATS + 8 * BQ;
  static constexpr int LDS_BYTES = NBUF * BUF_ELEMS * 2;
  static constexpr int DK = D / 16, DB = D / 32, NS = 2 * DB;
  static constexpr int NIW = TILE / 512 / WAVES;   // 1 KB loads per wave per tensor tile
  static_assert(DK == 2 * NIW && NS == DK, "one load every other k-step; B fits C's steps");
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int nkt, float c2,
    float scale) {
  using C = DkdvCfg<D>;
  constexpr int DK = C::DK, DB = C::DB, NS = C::NS, NIW = C::NIW;
  constexpr int RA = kDkdvReadAhead, SA = kDkdvStepAhead;
  constexpr int HPS = 8 / NS;                  // half-parts of B per step of C
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
  const int g = lane >> 5;
  const int key = kt * C::BK + wave * 32 + (lane & 31);   // this lane's key row

  // K and V rows of this lane's key as B operands (k-step kk: cols kk*16+8g..),
  // kept in accumulation registers (all loads are issued before any is used).
  bf16x8 kreg[DK], vreg[DK];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) {
    const uint32_t off = (uint32_t)((key * D + kk * 16 + g * 8) * 2);
    kreg[kk] = as_bf16x8(buf_load16(rk, off));
    vreg[kk] = as_bf16x8(buf_load16(rv, off));
  }
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) {
    asm volatile("" : "+a"(kreg[kk]));
    asm volatile("" : "+a"(vreg[kk]));
  }
  f32x16 dvt[DB], dkt[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) dvt[cb] = dkt[cb] = zero16();

  const int nqt = (N + C::BQ - 1) / C::BQ;
  const float neg_inv_scale = -1.0f / scale;
  // Load m (0 .. 2 NIW - 1) of this wave's share of tile `t` into buffer b;
  // with m == 0 each wave also loads the tile's LSE (even waves) or delta
  // (odd waves) row, waves 2 and 3 into the spare copy.
  static_assert(C::BQ == 64, "one wave per statistic");
  const uint32_t dvoff = tile_dma_voff<D, C::WAVES>(wave, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  auto dma = [&](int b, int t, int m) {
    const int tensor = m / NIW;
    tile_dma<D, C::WAVES>(lds0 + (uint32_t)((b * C::BUF_ELEMS + tensor * C::TILE) * 2),
                          tensor ? rdo : rq, dvoff, (uint32_t)(t * C::BQ * D * 2), wave, m % NIW);
    if (m == 0)
      lds_dma4((wave & 1) ? rdel : rlse, (uint32_t)(lane * 4),
               lds0 + (uint32_t)((b * C::BUF_ELEMS + C::OFF_STATS) * 2 + wave * C::BQ * 4),
               (uint32_t)(t * C::BQ * 4));
  };
  // B operand of the bias k-step: bf16 ones at k = 0, 1, 2 (lanes of k-group
  // 0), zeros elsewhere.
  bf16x8 ones3;
  {
    const u32x4 w = {g ? 0u : 0x3F803F80u, g ? 0u : 0x00003F80u, 0u, 0u};
    ones3 = as_bf16x8(w);
    asm volatile("" : "+a"(ones3));
  }
  // A operand of the bias k-step for value x: (hi, mid, lo, 0, ..) with
  // hi + mid + lo == x exactly (each part keeps the next 8 significand bits).
  auto split3 = [](float x) {
    const uint32_t hb = __float_as_uint(x) & 0xFFFF0000u;
    const float r1 = x - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(mb);
    const u32x4 w = {(hb >> 16) | mb, __float_as_uint(r2) >> 16, 0u, 0u};
    return as_bf16x8(w);
  };

  // This lane's LDS byte offsets: row operands and statistics in the buffer
  // the A phases read, transposing reads in the buffer the C phases read.
  // Both start at buffer 0 and advance once per tile.
  uint32_t ra[DK], rc[DB][2];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) ra[kk] = (uint32_t)(2 * row_read_off<D>(lane, kk));
  uint32_t ra_st = (uint32_t)(2 * C::OFF_STATS + 4 * (lane & 31));
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) {
    rc[cb][0] = (uint32_t)(2 * tr_read_off<D>(lane, cb, 0));
    rc[cb][1] = (uint32_t)(2 * tr_read_off<D>(lane, cb, 1));
  }
  auto at = [&](uint32_t byte_off) {
    return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(smem) + byte_off);
  };

  f32x16 s, dp;                  // S and dP of the latest A
  u32x4 pw[2][2], sw[2][2];      // P and dS of two blocks as bf16 pairs: [set][16-query half]

  // The first PF k-steps' operands of an A, and its query row's LSE and
  // delta, are read ahead (a_pre) during the preceding B|C phase.
  constexpr int PF = 2;
  static_assert(PF <= RA, "prefetch within the read-ahead window");
  bf16x8 pqa[PF], poa[PF];
  float plse, pdel;
  auto a_pre = [&](int qb) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      pqa[kk] = lds_bf16x8(at(ra[kk]) + qb * 32 * D + C::OFF_Q);
      poa[kk] = lds_bf16x8(at(ra[kk]) + qb * 32 * D + C::OFF_DO);
    }
    // This lane's query row qb*32 + lane%32: its LSE and delta.
    const float* st = reinterpret_cast<const float*>(at(ra_st)) + qb * 32;
    plse = st[0];
    pdel = st[C::BQ];
  };

  // A(block qb of the A buffer), after a_pre(qb), with loads m0 .. m0 + NIW
  // - 1 of tile tl into buffer bl when do_dma.
  auto a_phase = [&](int qb, bool do_dma, int bl, int tl, int m0) {
    const uint16_t* rp[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) rp[kk] = at(ra[kk]) + qb * 32 * D;
    const float lse_r = plse, del_r = pdel;
    s = zero16();
    dp = zero16();
    bf16x8 qa[RA + 1], oa[RA + 1];
#pragma unroll
    for (int kk = 0; kk < RA; ++kk) {
      if (kk < PF) {
        qa[kk] = pqa[kk];
        oa[kk] = poa[kk];
      } else {
        qa[kk] = lds_bf16x8(rp[kk] + C::OFF_Q);
        oa[kk] = lds_bf16x8(rp[kk] + C::OFF_DO);
      }
    }
    bf16x8 qbias, obias;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      if (kk + RA < DK) {
        qa[(kk + RA) % (RA + 1)] = lds_bf16x8(rp[kk + RA] + C::OFF_Q);
        oa[(kk + RA) % (RA + 1)] = lds_bf16x8(rp[kk + RA] + C::OFF_DO);
      }
      __builtin_amdgcn_sched_barrier(0);
      s = mfma32(qa[kk % (RA + 1)], kreg[kk], s);
      dp = mfma32(oa[kk % (RA + 1)], vreg[kk], dp);
      __builtin_amdgcn_sched_barrier(0);
      if (do_dma && (kk & 1) == 0) dma(bl, tl, m0 + (kk >> 1));
      if (kk == DK / 2) {
        __builtin_amdgcn_sched_barrier(0);
        qbias = split3(lse_r * neg_inv_scale);
        obias = split3(-del_r);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    s = mfma32(qbias, ones3, s);
    dp = mfma32(obias, ones3, dp);
    __builtin_amdgcn_sched_barrier(0);
  };

  // B of the latest A into P/dS set `bset`, interleaved with C(block cqb of
  // the C buffer, P/dS set 1 - bset) when do_c.  Half-part hp
  // covers score elements 4r + 2(hp&1) + {0,1}, r = hp/2; step n of C
  // finishes half-parts n*HPS .. (multiply, pack) and starts those of step
  // n+1 (scale, exp).  Three steps before the end, `pre` > 0 reads ahead for
  // the next A: pre == 1 first publishes the next tile (wait for this wave's
  // loads, barrier, move the A offsets on by `step`) and reads block 0 of
  // it; pre == 2 reads block 1 of the current A buffer.
  uint32_t step = 0;
  auto bc_phase = [&](int bset, bool do_c, int cqb, int pre) {
    float x[8][2];
    auto stage1a = [&](int hp) {   // scale
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        x[hp][e] = s[4 * (hp >> 1) + 2 * (hp & 1) + e] * c2;
        asm volatile("" : "+v"(x[hp][e]));
      }
    };
    auto stage1b = [&](int hp) {   // exp
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        x[hp][e] = fast_exp2(x[hp][e]);
        asm volatile("" : "+v"(x[hp][e]));
      }
    };
    float y[8][2];
    auto stage2a = [&](int hp) {   // dS = P dP'
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        y[hp][e] = x[hp][e] * dp[4 * (hp >> 1) + 2 * (hp & 1) + e];
        asm volatile("" : "+v"(y[hp][e]));
      }
    };
    auto stage2b = [&](int hp) {   // pack
      const int r = hp >> 1;
      uint32_t pv = pack_bf16x2(x[hp][0], x[hp][1]);
      uint32_t sv = pack_bf16x2(y[hp][0], y[hp][1]);
      asm volatile("" : "+v"(pv), "+v"(sv));
      pw[bset][r >> 1][2 * (r & 1) + (hp & 1)] = pv;
      sw[bset][r >> 1][2 * (r & 1) + (hp & 1)] = sv;
    };

    const uint16_t* tp[DB][2];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) tp[cb][h] = at(rc[cb][h]) + cqb * 32 * D;
    bf16x8 oa[SA + 1], qa[SA + 1];
    auto rd = [&](int n, bf16x8& o_, bf16x8& q_) {
      const int h = n / DB, cb = n % DB;
      o_ = tr_read2(tp[cb][0] + C::OFF_DO + h * 16 * D, tp[cb][1] + C::OFF_DO + h * 16 * D);
      q_ = tr_read2(tp[cb][0] + C::OFF_Q + h * 16 * D, tp[cb][1] + C::OFF_Q + h * 16 * D);
    };
    if (do_c) {
#pragma unroll
      for (int n = 0; n < SA; ++n) rd(n, oa[n], qa[n]);
    }
#pragma unroll
    for (int i = 0; i < HPS; ++i) stage1a(i);
#pragma unroll
    for (int i = 0; i < HPS; ++i) stage1b(i);
    const int cset = 1 - bset;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      if (do_c && n + SA < NS) rd(n + SA, oa[(n + SA) % (SA + 1)], qa[(n + SA) % (SA + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      const int h = n / DB, cb = n % DB;
      if (do_c) dvt[cb] = mfma32(oa[n % (SA + 1)], as_bf16x8(pw[cset][h]), dvt[cb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < HPS; ++i) {
        if (n + 1 < NS) stage1a((n + 1) * HPS + i);
        stage2a(n * HPS + i);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_c) dkt[cb] = mfma32(qa[n % (SA + 1)], as_bf16x8(sw[cset][h]), dkt[cb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < HPS; ++i) {
        if (n + 1 < NS) stage1b((n + 1) * HPS + i);
        stage2b(n * HPS + i);
      }
      if (pre > 0 && n == NS - 3) {
        __builtin_amdgcn_sched_barrier(0);
        if (pre == 1) {
          wait_vmem();       // this wave's loads of the next tile have landed
          __syncthreads();   // ... and everyone's; the tile before the current one is free
#pragma unroll
          for (int kk = 0; kk < DK; ++kk) ra[kk] += step;
          ra_st += step;
        }
        a_pre(pre == 1 ? 0 : 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: tile 0 published in buffer 0, tile 1 in flight to buffer 1,
  // A(0), B(0), A(1) done.
#pragma unroll
  for (int m = 0; m < 2 * NIW; ++m) dma(0, 0, m);
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 2 * NIW; ++m) dma(1, 1, m);
  a_pre(0);
  a_phase(0, false, 0, 0, 0);
  bc_phase(0, false, 0, 2);
  a_phase(1, false, 0, 0, 0);

  int b0 = 0, b1 = 1, b2 = 2;   // buffers of tiles t, t+1, t+2
  for (int t = 0; t < nqt; ++t) {
    step = (uint32_t)((b1 - b0) * C::BUF_ELEMS * 2);   // next buffer, mod 2^32
    bc_phase(1, true, 0, 1);                   // B(2t+1) | C(2t); publishes tile t+1
    a_phase(0, true, b2, t + 2, 0);            // A(2t+2), first half of tile t+2's loads
    bc_phase(0, true, 1, 2);                   // B(2t+2) | C(2t+1)
    a_phase(1, true, b2, t + 2, NIW);          // A(2t+3), second half
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {          // C phases move on to tile t+1
      rc[cb][0] += step;
      rc[cb][1] += step;
    }
    b0 = b1;
    b1 = b2;
    b2 = b2 == 2 ? 0 : b2 + 1;
  }
  wait_vmem();   // no direct loads left in flight at exit

  // dV^T / dK^T element i of block cb: column cb*32 + 8*(i/4) + 4g + i%4 of
  // this lane's key row.
  if (key < N) {
    uint16_t* dkr = dk + hoff + (int64_t)key * D;
    uint16_t* dvr = dv + hoff + (int64_t)key * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
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
// dQ: workgroup owns 256 queries (8 waves x 32, two per SIMD), loops over
// 64-key tiles; each K/V tile in LDS serves all 256 queries.  A wave raises
// its priority while it issues matrix-core instructions, so that the other
// wave of its SIMD runs its vector work in between.
// The contractions use the 16 x 16 x 32 instruction (device_common.h): a
// wave owns two 16-query blocks, and lane l holds query l%16 of each block
// for keys 4(l/16) + 0..3 of every 16 keys.  Per wave and 32-key block:
//   S^T  = K Q^T    (A = K rows from LDS, B = Q regs)
//   dP^T = V dO^T   (A = V rows from LDS, B = dO regs)
//   P^T = 2^(c S^T - LSE log2 e), dS^T = P^T (dP^T - D)   (per-query stats)
//   dQ^T += K^T dS^T (A = K^T from LDS, B = dS^T from the accumulators)
// K and V tiles are in row-segment order (lds_tile.h): K is read along rows
// for S^T and with transposing reads for K^T, V along rows only, and the
// tiles' swizzle keeps both kinds of read free of bank conflicts.  Keys past
// N read as zero rows of K and V and their scores are set to -inf, so their
// P and dS are 0.
// ---------------------------------------------------------------------------
template <int D>
struct DqCfg {
  static constexpr int BQ = 256, BK = 64, WAVES = 8, THREADS = 64 * WAVES;
  static constexpr int TILE = BK * D;          // one K or V tile (bf16)
  static constexpr int BUF_ELEMS = 2 * TILE;   // K tile then V tile
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int DK = D / 32, DB = D / 16;
};

template <int D, int RA = kReadAhead, int SA = kStepAhead>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int N, int nqt, float c2, float scale) {
  using C = DqCfg<D>;
  static_assert(RA <= 2 * C::DK && SA <= C::DB, "read-ahead within one block's operands");
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
  const int li = lane & 15, g = lane >> 4;
  const int qrow0 = qt * C::BQ + wave * 32 + li;   // rows qrow0 and qrow0 + 16

  bf16x8 qreg[2][C::DK], oreg[2][C::DK];
  float lse2[2], dl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qrow0 + 16 * qb;
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk) {
      const uint32_t off = (uint32_t)((qrow * D + kk * 32 + g * 8) * 2);
      qreg[qb][kk] = as_bf16x8(buf_load16(rq, off));
      oreg[qb][kk] = as_bf16x8(buf_load16(rdo, off));
    }
    lse2[qb] = qrow < N ? lse[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
    dl[qb] = qrow < N ? delta[(int64_t)bh * N + qrow] : 0.0f;
  }

  f32x4 dqt[2][C::DB];   // dQ^T blocks: lane l holds columns 16 db + 4 g + 0..3
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) dqt[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nkt = (N + C::BK - 1) / C::BK;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t voff = seg_dma_voff<D, C::WAVES>(wave, lane);
  constexpr int NU = (C::BK / 16) * (D / 32) / C::WAVES;
  static_assert(NU * C::WAVES == (C::BK / 16) * (D / 32), "whole loads per wave");
  auto load_tile = [&](int jt, int b) {
    uint32_t kd = lds0 + (uint32_t)(b * C::BUF_ELEMS * 2), vd = kd + (uint32_t)(C::TILE * 2);
    const uint32_t r0 = (uint32_t)(jt * C::BK * D * 2);
    asm volatile("" : "+s"(kd), "+s"(vd));   // one address per buffer, not one per load
#pragma unroll
    for (int u = 0; u < NU; ++u) seg_dma<D, C::WAVES>(kd, rk, voff, r0, wave, u);
#pragma unroll
    for (int u = 0; u < NU; ++u) seg_dma<D, C::WAVES>(vd, rv, voff, r0, wave, u);
  };
  const uint32_t rowop = seg_rowop16_base(lane);
  const uint32_t ktr0 = seg_trop16_base(lane, 0), ktr1 = seg_trop16_base(lane, 1);
  load_tile(0, 0);
  wait_vmem();
  __syncthreads();

  // One key tile; `ragged` (a compile-time flag) is set only for a last tile
  // that holds keys past N, so that the full tiles carry no masking code.
  auto tile = [&](int it, auto ragged) {
    uint32_t bo = (uint32_t)((it & 1) * C::BUF_ELEMS * 2);
    asm volatile("" : "+s"(bo));
    const uint8_t* kt8 = reinterpret_cast<const uint8_t*>(smem) + bo;
    const uint8_t* vt8 = kt8 + C::TILE * 2;
    const uint8_t* ktr[2] = {kt8 + ktr0, kt8 + ktr1};
    if (it + 1 < nkt) load_tile(it + 1, (it + 1) & 1);

    // One 32-key block at a time: S^T = K Q^T and dP^T = V dO^T over
    // operands n = (k-step n / 2, 16-key half n % 2), then P^T and dS^T in
    // the B-operand order of dQ^T += K^T dS^T, then that contraction with
    // K^T gathered by transposing reads.
#pragma unroll
    for (int kb2 = 0; kb2 < C::BK / 32; ++kb2) {
      f32x4 s[2][2], dp[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[qb][h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          dp[qb][h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      {
        constexpr int NS = 2 * C::DK;
        auto rd = [&](const uint8_t* base, int n) {
          return *reinterpret_cast<const bf16x8*>(
              base + seg_rowop16_imm<D>(2 * kb2 + n % 2, n / 2));
        };
        bf16x8 ka[RA + 1], va[RA + 1];
#pragma unroll
        for (int n = 0; n < RA; ++n) {
          ka[n] = rd(kt8 + rowop, n);
          va[n] = rd(vt8 + rowop, n);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          if (n + RA < NS) {
            ka[(n + RA) % (RA + 1)] = rd(kt8 + rowop, n + RA);
            va[(n + RA) % (RA + 1)] = rd(vt8 + rowop, n + RA);
          }
          __builtin_amdgcn_sched_barrier(0);
          const int kk = n / 2, h = n % 2;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            s[qb][h] = mfma16(ka[n % (RA + 1)], qreg[qb][kk], s[qb][h]);
            dp[qb][h] = mfma16(va[n % (RA + 1)], oreg[qb][kk], dp[qb][h]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
      // Keys past N in the last tile read as zero rows of K and V; their P
      // would be 2^(-LSE log2 e), which overflows when every score of the
      // row is below about -88.  They do not exist: their scores are -inf,
      // so P and dS are 0.
      if constexpr (decltype(ragged)::value) {
        const int key0 = it * C::BK + kb2 * 32;
        if (key0 + 32 > N) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (key0 + 16 * h + 4 * g + i >= N) s[qb][h][i] = -INFINITY;
        }
      }
      bf16x8 sb[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        u32x4 sw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int h = e >> 1, i = 2 * (e & 1);
          const float p0 = fast_exp2(fmaf(s[qb][h][i], c2, -lse2[qb]));
          const float p1 = fast_exp2(fmaf(s[qb][h][i + 1], c2, -lse2[qb]));
          sw[e] = pack_bf16x2(p0 * (dp[qb][h][i] - dl[qb]), p1 * (dp[qb][h][i + 1] - dl[qb]));
        }
        sb[qb] = as_bf16x8(sw);
      }
      {
        bf16x8 ka[SA + 1];
#pragma unroll
        for (int n = 0; n < SA; ++n) ka[n] = seg_trop16_read<D>(ktr[n & 1], kb2, n);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          if (db + SA < C::DB)
            ka[(db + SA) % (SA + 1)] = seg_trop16_read<D>(ktr[(db + SA) & 1], kb2, db + SA);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            dqt[qb][db] = mfma16(ka[db % (SA + 1)], sb[qb], dqt[qb][db]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }

    wait_vmem();
    __syncthreads();
  };
  const int nfull = N / C::BK;   // tiles whose keys are all < N
  for (int it = 0; it < nfull; ++it) tile(it, std::false_type{});
  if (nfull < nkt) tile(nfull, std::true_type{});

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qrow0 + 16 * qb;
    if (qrow < N) {
      uint16_t* dqr = dq + hoff + (int64_t)qrow * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        u32x2 w;
        w[0] = pack_bf16x2(dqt[qb][db][0] * scale, dqt[qb][db][1] * scale);
        w[1] = pack_bf16x2(dqt[qb][db][2] * scale, dqt[qb][db][3] * scale);
        *reinterpret_cast<u32x2*>(dqr + db * 16 + 4 * g) = w;
      }
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
  // Chunks of whole blocks of RPB rows.
  return launch_in_chunks((rows + RPB - 1) / RPB, 256, [&](int64_t b0, int64_t nb) {
    const int64_t r0 = b0 * RPB, nr = std::min(nb * RPB, rows - r0);
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)nb), dim3(256), 0, stream, o + r0 * D,
                       dO + r0 * D, delta + r0, nr);
    return (int)hipGetLastError();
  });
}

template <int D>
int launch_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                const uint16_t* dO, const float* delta, uint16_t* dk, uint16_t* dv, int64_t BH,
                int64_t N, float scale, hipStream_t stream) {
  using C = DkdvCfg<D>;
  const int nkt = (int)((N + C::BK - 1) / C::BK);
  const int64_t per_head = (int64_t)nkt * C::THREADS;
  if (!unit_fits(per_head)) return kErrGridTooLarge;
  hipError_t e = allow_lds(bwd_dkdv_kernel<D>, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  return launch_in_chunks(BH, per_head, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * D, roff = h0 * N;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(nkt * nh)), dim3(C::THREADS),
                       C::LDS_BYTES, stream, q + off, k + off, v + off, lse + roff, dO + off,
                       delta + roff, dk + off, dv + off, (int)N, nkt, scale * kLog2e, scale);
    return (int)hipGetLastError();
  });
}

template <int D, int RA = kReadAhead, int SA = kStepAhead>
int launch_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                const uint16_t* dO, const float* delta, uint16_t* dq, int64_t BH, int64_t N,
                float scale, hipStream_t stream) {
  using C = DqCfg<D>;
  const int nqt = (int)((N + C::BQ - 1) / C::BQ);
  const int64_t per_head = (int64_t)nqt * C::THREADS;
  if (!unit_fits(per_head)) return kErrGridTooLarge;
  hipError_t e = allow_lds(bwd_dq_kernel<D, RA, SA>, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  return launch_in_chunks(BH, per_head, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * D, roff = h0 * N;
    hipLaunchKernelGGL((bwd_dq_kernel<D, RA, SA>), dim3((unsigned)(nqt * nh)),
                       dim3(C::THREADS), C::LDS_BYTES, stream, q + off, k + off, v + off,
                       lse + roff, dO + off, delta + roff, dq + off, (int)N, nqt,
                       scale * kLog2e, scale);
    return (int)hipGetLastError();
  });
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
