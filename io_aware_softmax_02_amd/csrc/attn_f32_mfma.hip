// fp32 attention on the matrix cores (v_mfma_f32_32x32x2_f32) for head dims
// 64 and 128.  Same method as the bf16 forward (账房先生的奔命, section 六:
// tiles of Q, K and V; rescale identity of the star-observatory fable page,
// section "兩大核心魔法"; only O and the row statistic are written back,
// 算珠楼的掌簿人, 技术解读), with every operand and every intermediate in
// fp32: no rounding of P.
//
// Matrix-core layout of v_mfma_f32_32x32x2_f32: operand lane l holds row (A)
// or column (B) l % 32 at k = l / 32 (one value), the accumulator holds
// column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4 in element i.
// Contraction over d: lane group g = l / 32 covers d in [g D/2, (g+1) D/2),
// one column per instruction, so a lane's operands for four consecutive
// instructions are four consecutive floats (one 16-byte read).
// Scores are formed transposed, S^T = K Q^T: a lane owns one query row, and
// accumulator element i of a 32-key block is key 8 (i / 4) + 4 g + i % 4,
// which is exactly the B operand of O^T += V^T P^T at k-step i.  The V^T
// operand is read one float at a time from the V tile's column.
//
// LDS tiles (fp32, rows padded): K rows of D + 4 floats, so the 16-byte reads
// of 16 consecutive keys at one column fall on 16 different bank groups; V
// rows of D + 8 floats, so the column reads of two lane groups (keys 4 apart)
// fall on opposite halves of the 64 banks.  Tiles are staged through
// registers one tile ahead (zero past N) and double-buffered; one barrier per
// tile.
#include "device_common.h"
#include "launch_chunks.h"

namespace fa {
namespace {

constexpr float kSlackF32 = 8.0f;   // lazy-rescale slack, log2 units

__device__ __forceinline__ f32x16 mfma32f(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
struct F32Cfg {
  static constexpr int WAVES = 4, THREADS = 64 * WAVES, BR = 32 * WAVES, BC = 32;
  static constexpr int KS = D + 4;                 // K tile row stride (floats)
  static constexpr int VS = D + 8;                 // V tile row stride (floats)
  static constexpr int KT = BC * KS, VT = BC * VS;
  static constexpr int BUF = KT + VT;              // one buffer (floats)
  static constexpr int LDS_BYTES = 2 * BUF * 4;
  static constexpr int HK = D / 2;                 // k-steps per lane group
  static constexpr int DB = D / 32;                // 32-column blocks of O
  static constexpr int LOADS = BC * D / 4 / THREADS;   // 16-byte loads per thread per tile
  static_assert(LOADS >= 1 && BC * D / 4 % THREADS == 0, "whole loads per thread");
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_f32_mfma_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int N, int ntq, float c2) {
  using C = F32Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) float sm[];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / ntq, qt = logical - bh * ntq;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint32_t hbytes = (uint32_t)N * D * 4;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes);
  const rsrc_t rk = make_rsrc(k + hoff, hbytes);
  const rsrc_t rv = make_rsrc(v + hoff, hbytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int qrow = qt * C::BR + wave * 32 + li;

  // Q^T operands: k-step kk of this lane is column HK*g + kk of its query row.
  float qreg[C::HK];
#pragma unroll
  for (int j = 0; j < C::HK / 4; ++j) {
    const u32x4 w = buf_load16(rq, (uint32_t)((qrow * D + C::HK * g + 4 * j) * 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) qreg[4 * j + t] = __uint_as_float(w[t]);
  }
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.0f;

  // Tile staging: load u of this thread covers 16-byte chunk c = tid + 256 u
  // of the tile, row c / (D/4), column 4 (c % (D/4)).
  u32x4 kr[C::LOADS], vr[C::LOADS];
  auto load_regs = [&](int key0) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = tid + C::THREADS * u, row = c / (D / 4), col = 4 * (c % (D / 4));
      const uint32_t off = (uint32_t)(((key0 + row) * D + col) * 4);
      kr[u] = buf_load16(rk, off);
      vr[u] = buf_load16(rv, off);
    }
  };
  auto store_tile = [&](float* buf) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = tid + C::THREADS * u, row = c / (D / 4), col = 4 * (c % (D / 4));
      *reinterpret_cast<u32x4*>(buf + row * C::KS + col) = kr[u];
      *reinterpret_cast<u32x4*>(buf + C::KT + row * C::VS + col) = vr[u];
    }
  };

  const int nkt = (N + C::BC - 1) / C::BC;
  load_regs(0);
  store_tile(sm);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const float* Kt = sm + (j & 1) * C::BUF;
    const float* Vt = Kt + C::KT;
    if (j + 1 < nkt) load_regs((j + 1) * C::BC);

    // S^T = K_j Q^T: A = this lane's key row (li) at columns HK*g + kk.
    f32x16 s = zero16();
    const float* kl = Kt + li * C::KS + C::HK * g;
#pragma unroll
    for (int j4 = 0; j4 < C::HK / 4; ++j4) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(kl + 4 * j4);
#pragma unroll
      for (int t = 0; t < 4; ++t) s = mfma32f(kv[t], qreg[4 * j4 + t], s);
    }
    // Keys past N do not exist: their scores are -inf.
    if (j * C::BC + C::BC > N) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = j * C::BC + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= N) s[i] = -INFINITY;
      }
    }

    // Online softmax with a lazily moved reference (as in the bf16 forward):
    // P~ = 2^(c s - m_run) <= 2^kSlackF32; U and l share the reference.
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = max_across_halves(mx);
    const float m_cand = mx * c2;
    if (__any(m_cand > m_run + kSlackF32)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = fast_exp2(m_run - m_new);   // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      m_run = m_new;
    }
    float p[16], rs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(fmaf(s[i], c2, -m_run));
      rs += p[i];
    }
    l_run += rs;

    // O^T += V_j^T P^T: k-step kk is key 8 (kk/4) + 4 g + kk % 4, whose
    // probability is p[kk]; the V^T operand is that key's value at column
    // 32 db + li.
    const float* vl = Vt + 4 * g * C::VS + li;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        acc[db] = mfma32f(vl[(8 * (kk >> 2) + (kk & 3)) * C::VS + 32 * db], p[kk], acc[db]);

    if (j + 1 < nkt) store_tile(sm + ((j + 1) & 1) * C::BUF);
    __syncthreads();   // tile j+1 published; tile j no longer read
  }

  // Epilogue: O = U / l; element i of block db is column 32 db + 8 (i/4) +
  // 4 g + i%4 of this lane's query row.
  const float l_tot = sum_across_halves(l_run);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    float* orow = o + hoff + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * r + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r + 4 * g) = w;
      }
    if (g == 0) lse[(int64_t)bh * N + qrow] = kLn2 * (m_run + log2f(l_tot));
  }
}

template <int D>
int launch_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int64_t BH,
               int64_t N, float scale, hipStream_t stream) {
  using C = F32Cfg<D>;
  const int ntq = (int)((N + C::BR - 1) / C::BR);
  const int64_t per_head = (int64_t)ntq * C::THREADS;
  if (!unit_fits(per_head)) return kErrGridTooLarge;
  auto kern = fwd_f32_mfma_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  return launch_in_chunks(BH, per_head, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * D;
    hipLaunchKernelGGL(kern, dim3((unsigned)(ntq * nh)), dim3(C::THREADS), C::LDS_BYTES, stream,
                       q + off, k + off, v + off, o + off, lse + h0 * N, (int)N, ntq,
                       scale * kLog2e);
    return (int)hipGetLastError();
  });
}

// ---------------------------------------------------------------------------
// Backward (账房先生的奔命, section 七: P recomputed from Q, K and the saved
// LSE).  Two kernels, as for bf16: dK/dV with keys resident, dQ with queries
// resident (no atomics).  Tiles of 32 rows of the streamed tensors, padded
// rows of D + 4 floats, staged through registers one tile ahead.
// ---------------------------------------------------------------------------
template <int D>
struct F32BwdCfg {
  static constexpr int WAVES = 4, THREADS = 64 * WAVES, BRES = 32 * WAVES, BT = 32;
  static constexpr int S = D + 4;                  // tile row stride (floats)
  static constexpr int T = BT * S;                 // one tile (floats)
  static constexpr int BUF = 2 * T + 2 * BT;       // two tiles + two per-row statistics
  static constexpr int LDS_BYTES = 2 * BUF * 4;
  static constexpr int HK = D / 2, DB = D / 32;
  static constexpr int LOADS = BT * D / 4 / THREADS;
};

// dK / dV: each wave owns 32 keys (lane: key li of the wave's block); per
// 32-query tile (accumulator element i of a tile is query 8 (i/4) + 4 g + i%4):
//   S = Q K^T, dP = dO V^T        (A = Q / dO rows from LDS, B = K / V regs)
//   P = 2^(c S - LSE log2 e), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS (A = dO / Q columns from LDS, B = P / dS)
// Query rows past N are zero rows of Q and dO with LSE = D = 0: their P
// multiplies a zero dO row and their dS is 0.
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_f32_mfma_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dO,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv, int N,
    int nkt, float c2, float scale) {
  using C = F32BwdCfg<D>;
  extern __shared__ __attribute__((aligned(16))) float sm[];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nkt, kt = logical - bh * nkt;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint32_t hbytes = (uint32_t)N * D * 4;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes);
  const rsrc_t rdo = make_rsrc(dO + hoff, hbytes);
  const rsrc_t rk = make_rsrc(k + hoff, hbytes);
  const rsrc_t rv = make_rsrc(v + hoff, hbytes);
  const rsrc_t rl = make_rsrc(lse + (int64_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rd = make_rsrc(delta + (int64_t)bh * N, (uint32_t)N * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int key = kt * C::BRES + wave * 32 + li;

  float kreg[C::HK], vreg[C::HK];
#pragma unroll
  for (int j = 0; j < C::HK / 4; ++j) {
    const uint32_t off = (uint32_t)((key * D + C::HK * g + 4 * j) * 4);
    const u32x4 a = buf_load16(rk, off), b = buf_load16(rv, off);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kreg[4 * j + t] = __uint_as_float(a[t]);
      vreg[4 * j + t] = __uint_as_float(b[t]);
    }
  }
  f32x16 dvt[C::DB], dkt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dvt[db] = dkt[db] = zero16();

  u32x4 qr[C::LOADS], gr[C::LOADS];
  float st = 0.0f;
  auto load_regs = [&](int r0) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = tid + C::THREADS * u, row = c / (D / 4), col = 4 * (c % (D / 4));
      const uint32_t off = (uint32_t)(((r0 + row) * D + col) * 4);
      qr[u] = buf_load16(rq, off);
      gr[u] = buf_load16(rdo, off);
    }
    if (wave == 0) {   // lanes 0..31: LSE, 32..63: delta (both loaded, no divergent source)
      const uint32_t off = (uint32_t)((r0 + (lane & 31)) * 4);
      const float a = buf_loadf(rl, off), b = buf_loadf(rd, off);
      st = lane < 32 ? a : b;
    }
  };
  auto store_tile = [&](float* buf) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = tid + C::THREADS * u, row = c / (D / 4), col = 4 * (c % (D / 4));
      *reinterpret_cast<u32x4*>(buf + row * C::S + col) = qr[u];
      *reinterpret_cast<u32x4*>(buf + C::T + row * C::S + col) = gr[u];
    }
    static_assert(2 * C::BT == 64, "one wave carries the statistics");
    if (wave == 0) buf[2 * C::T + lane] = lane < 32 ? st * kLog2e : st;   // LSE log2 units, delta
  };

  const int nqt = (N + C::BT - 1) / C::BT;
  load_regs(0);
  store_tile(sm);
  __syncthreads();

  for (int it = 0; it < nqt; ++it) {
    const float* Qt = sm + (it & 1) * C::BUF;
    const float* Gt = Qt + C::T;
    const float* stats = Qt + 2 * C::T;
    if (it + 1 < nqt) load_regs((it + 1) * C::BT);

    f32x16 s = zero16(), dp = zero16();
    const float* ql = Qt + li * C::S + C::HK * g;
    const float* gl = Gt + li * C::S + C::HK * g;
#pragma unroll
    for (int j4 = 0; j4 < C::HK / 4; ++j4) {
      const f32x4 qv = *reinterpret_cast<const f32x4*>(ql + 4 * j4);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gl + 4 * j4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s = mfma32f(qv[t], kreg[4 * j4 + t], s);
        dp = mfma32f(gv[t], vreg[4 * j4 + t], dp);
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(stats + 8 * r + 4 * g);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(stats + C::BT + 8 * r + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[4 * r + e] = fast_exp2(fmaf(s[4 * r + e], c2, -l4[e]));
        ds[4 * r + e] = p[4 * r + e] * (dp[4 * r + e] - d4[e]);
      }
    }
    // k-step kk: query 8 (kk/4) + 4 g + kk % 4, column 32 db + li.
    const float* gc = Gt + 4 * g * C::S + li;
    const float* qc = Qt + 4 * g * C::S + li;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int o = (8 * (kk >> 2) + (kk & 3)) * C::S + 32 * db;
        dvt[db] = mfma32f(gc[o], p[kk], dvt[db]);
        dkt[db] = mfma32f(qc[o], ds[kk], dkt[db]);
      }

    if (it + 1 < nqt) store_tile(sm + ((it + 1) & 1) * C::BUF);
    __syncthreads();
  }

  // element i of block db: column 32 db + 8 (i/4) + 4 g + i%4 of this lane's key row
  if (key < N) {
    float* dkr = dk + hoff + (int64_t)key * D;
    float* dvr = dv + hoff + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dkt[db][4 * r + e] * scale;
          b[e] = dvt[db][4 * r + e];
        }
        *reinterpret_cast<f32x4*>(dkr + 32 * db + 8 * r + 4 * g) = a;
        *reinterpret_cast<f32x4*>(dvr + 32 * db + 8 * r + 4 * g) = b;
      }
  }
}

// dQ: each wave owns 32 queries (lane: query li); per 32-key tile
// (accumulator element i is key 8 (i/4) + 4 g + i%4):
//   S^T = K Q^T, dP^T = V dO^T     (A = K / V rows from LDS, B = Q / dO regs)
//   P^T = 2^(c S^T - LSE log2 e), dS^T = P^T (dP^T - D)   (lane-uniform stats)
//   dQ^T += K^T dS^T               (A = K columns from LDS, B = dS^T)
// Keys past N are zero rows of K and V; their dS meets a zero K row.
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_f32_mfma_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dO,
    const float* __restrict__ delta, float* __restrict__ dq, int N, int nqt, float c2,
    float scale) {
  using C = F32BwdCfg<D>;
  extern __shared__ __attribute__((aligned(16))) float sm[];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt, qt = logical - bh * nqt;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint32_t hbytes = (uint32_t)N * D * 4;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes);
  const rsrc_t rdo = make_rsrc(dO + hoff, hbytes);
  const rsrc_t rk = make_rsrc(k + hoff, hbytes);
  const rsrc_t rv = make_rsrc(v + hoff, hbytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int qrow = qt * C::BRES + wave * 32 + li;

  float qreg[C::HK], oreg[C::HK];
#pragma unroll
  for (int j = 0; j < C::HK / 4; ++j) {
    const uint32_t off = (uint32_t)((qrow * D + C::HK * g + 4 * j) * 4);
    const u32x4 a = buf_load16(rq, off), b = buf_load16(rdo, off);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qreg[4 * j + t] = __uint_as_float(a[t]);
      oreg[4 * j + t] = __uint_as_float(b[t]);
    }
  }
  const float lse2 = qrow < N ? lse[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dl = qrow < N ? delta[(int64_t)bh * N + qrow] : 0.0f;
  f32x16 dqt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqt[db] = zero16();

  u32x4 kr[C::LOADS], vr[C::LOADS];
  auto load_regs = [&](int r0) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = tid + C::THREADS * u, row = c / (D / 4), col = 4 * (c % (D / 4));
      const uint32_t off = (uint32_t)(((r0 + row) * D + col) * 4);
      kr[u] = buf_load16(rk, off);
      vr[u] = buf_load16(rv, off);
    }
  };
  auto store_tile = [&](float* buf) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = tid + C::THREADS * u, row = c / (D / 4), col = 4 * (c % (D / 4));
      *reinterpret_cast<u32x4*>(buf + row * C::S + col) = kr[u];
      *reinterpret_cast<u32x4*>(buf + C::T + row * C::S + col) = vr[u];
    }
  };

  const int nkt = (N + C::BT - 1) / C::BT;
  load_regs(0);
  store_tile(sm);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const float* Kt = sm + (j & 1) * C::BUF;
    const float* Vt = Kt + C::T;
    if (j + 1 < nkt) load_regs((j + 1) * C::BT);

    f32x16 s = zero16(), dp = zero16();
    const float* kl = Kt + li * C::S + C::HK * g;
    const float* vl = Vt + li * C::S + C::HK * g;
#pragma unroll
    for (int j4 = 0; j4 < C::HK / 4; ++j4) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(kl + 4 * j4);
      const f32x4 vv = *reinterpret_cast<const f32x4*>(vl + 4 * j4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s = mfma32f(kv[t], qreg[4 * j4 + t], s);
        dp = mfma32f(vv[t], oreg[4 * j4 + t], dp);
      }
    }
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = fast_exp2(fmaf(s[i], c2, -lse2)) * (dp[i] - dl);
    // Keys past N in the last tile read as zero rows of K and V; their P
    // would be 2^(-LSE log2 e), which overflows when every score of the row
    // is below about -88.  They do not exist, so their dS is 0.
    if (j * C::BT + C::BT > N) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (j * C::BT + 8 * (i >> 2) + 4 * g + (i & 3) >= N) ds[i] = 0.0f;
    }
    const float* kc = Kt + 4 * g * C::S + li;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        dqt[db] = mfma32f(kc[(8 * (kk >> 2) + (kk & 3)) * C::S + 32 * db], ds[kk], dqt[db]);

    if (j + 1 < nkt) store_tile(sm + ((j + 1) & 1) * C::BUF);
    __syncthreads();
  }

  if (qrow < N) {
    float* dqr = dq + hoff + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = dqt[db][4 * r + e] * scale;
        *reinterpret_cast<f32x4*>(dqr + 32 * db + 8 * r + 4 * g) = a;
      }
  }
}

template <int D>
int launch_bwd(const float* q, const float* k, const float* v, const float* lse,
               const float* dO, const float* delta, float* dq, float* dk, float* dv, int64_t BH,
               int64_t N, float scale, hipStream_t stream) {
  using C = F32BwdCfg<D>;
  const int nt = (int)((N + C::BRES - 1) / C::BRES);
  const int64_t per_head = (int64_t)nt * C::THREADS;
  if (!unit_fits(per_head)) return kErrGridTooLarge;
  auto kd = bwd_dkdv_f32_mfma_kernel<D>;
  auto kq = bwd_dq_f32_mfma_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kd,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  e = hipFuncSetAttribute((const void*)kq, hipFuncAttributeMaxDynamicSharedMemorySize,
                          C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  const int r = launch_in_chunks(BH, per_head, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * D, roff = h0 * N;
    hipLaunchKernelGGL(kd, dim3((unsigned)(nt * nh)), dim3(C::THREADS), C::LDS_BYTES, stream,
                       q + off, k + off, v + off, lse + roff, dO + off, delta + roff, dk + off,
                       dv + off, (int)N, nt, scale * kLog2e, scale);
    return (int)hipGetLastError();
  });
  if (r != 0) return r;
  return launch_in_chunks(BH, per_head, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * D, roff = h0 * N;
    hipLaunchKernelGGL(kq, dim3((unsigned)(nt * nh)), dim3(C::THREADS), C::LDS_BYTES, stream,
                       q + off, k + off, v + off, lse + roff, dO + off, delta + roff, dq + off,
                       (int)N, nt, scale * kLog2e, scale);
    return (int)hipGetLastError();
  });
}

}  // namespace

int launch_bwd_f32_mfma(const float* q, const float* k, const float* v, const float* lse,
                        const float* dO, const float* delta, float* dq, float* dk, float* dv,
                        int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream) {
  return d == 128 ? launch_bwd<128>(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, scale, stream)
                  : launch_bwd<64>(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, scale, stream);
}

// Whether the matrix-core fp32 kernels can take this shape: d of 64 or 128
// and one head of one tensor (plus a tile past the end) within 32-bit offsets.
bool f32_mfma_fits(int64_t N, int64_t d) {
  return (d == 64 || d == 128) && (N + 64) * d * 4 < (int64_t(1) << 31);
}

int launch_fwd_f32_mfma(const float* q, const float* k, const float* v, float* o, float* lse,
                        int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream) {
  return d == 128 ? launch_fwd<128>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_fwd<64>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
