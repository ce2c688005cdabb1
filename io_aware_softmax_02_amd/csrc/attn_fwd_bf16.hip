// bf16 attention forward for gfx950: one fused kernel, matrix cores for the
// two contractions, online softmax in registers.
//
// Method (page tags: 账房先生的奔命 = carrie-l.github.io; star-observatory
// fable = ckw19810413.github.io; 算珠楼的掌簿人 = hespethorn.github.io):
//   Q is cut into row tiles and K, V into key tiles (账房先生的奔命, section 六,
//   "Tiling").  For each key tile the scores S = Q K_j^T live only in
//   registers; the running max m, running sum l and the unnormalised output
//   U are updated with the rescale factor 2^(m_old - m_new) (the identity
//   e^{x-m_new} = e^{x-m_old} e^{m_old-m_new} of the star-observatory fable,
//   section "兩大核心魔法"), and at the end O = U / l and LSE = m + ln l are
//   the only values written back (算珠楼的掌簿人, 技术解读).  Two sums are
//   kept: l in fp32 for the LSE, and the sum of the bf16-rounded weights U
//   was accumulated with, which O is divided by (so O is a convex
//   combination of V rows in the arithmetic performed).
//
// Work decomposition:
//   workgroup = NWAVES waves; each wave owns QB blocks of 32 query rows of one
//   (batch, head).  Key tiles of BC rows stream through LDS, double-buffered:
//   direct buffer->LDS loads of tile j+1 are issued at the start of tile j
//   (no registers involved), one barrier per tile.  With QB = 2 every K and V
//   operand read from LDS would feed two matrix-core instructions; the
//   instantiations below use QB = 1 and more waves, which measured faster.
//   Scores are formed transposed, S^T = K Q^T, so that each lane owns one
//   query row: lane l holds query l%32 for 16 of every 32 keys (the other 16
//   sit in lane l^32).  Row sums are in-lane; the row max, taken only when
//   the softmax reference has to move, is an in-lane reduction plus one
//   exchange between the two half-waves.  The probabilities leave the
//   score accumulators already in the B-operand layout of O^T += V^T P^T, so
//   P never touches LDS; the V^T operand is gathered from the V tile with
//   transposing LDS reads in the matching key order.  Both tiles are stored
//   in row-segment order (lds_tile.h): every direct load reads whole 64-byte
//   row segments, the rate at which the load path runs at full speed, and
//   every LDS read is a base register (two for K) plus an immediate offset,
//   free of bank conflicts.
//   Base-2 domain: c = scale * log2(e); p = 2^(c s - m) with m in log2 units;
//   LSE = ln 2 * (m + log2 l).
//
// Split-KV mode (SPLIT): the key tiles are cut into nsplit contiguous ranges
// and each workgroup handles one range of one query tile, writing that
// range's own normalised output (fp32) and LSE.  The ranges are recombined
// by the merge kernel (attn_merge.hip) with the same rescale identity.
#include "lds_tile.h"

namespace fa {
namespace {

// Slack of the lazily updated softmax reference, in log2 units.
constexpr float kSlack = 8.0f;
constexpr float kSlackPow = 256.0f;   // 2^kSlack
// k-steps of K operands, and (t, db) steps of V^T operands, read from LDS
// ahead of their use.
constexpr int kReadAhead = 2;
constexpr int kStepAhead = 4;

template <int D, int QB, int BC, int NWAVES = 4>
struct FwdCfg {
  static constexpr int WAVES = NWAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = WAVES * 32 * QB;      // query rows per workgroup
  static constexpr int KB = BC / 32;              // 32-key blocks per tile
  static constexpr int TILE = BC * D;             // one K or V tile (bf16), swizzled
  static constexpr int BUF_ELEMS = 2 * TILE;      // K tile then V tile
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int DK = D / 16;               // k-steps of the QK^T contraction
  static constexpr int DB = D / 32;               // 32-column blocks of O
  static_assert(BC % 32 == 0 && BC <= 128, "key tile is a multiple of 32 rows");
};

template <int D, int QB, int BC, int MINW, bool PRIO, int NWAVES = 4, bool SPLIT = false>
__global__ __launch_bounds__(64 * NWAVES, MINW) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o, float* __restrict__ lse, int N,
    int ntq, float c2, int nsplit, int64_t part_rows) {
  using C = FwdCfg<D, QB, BC, NWAVES>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  // Logical id = ((bh * nsplit) + p) * ntq + qt: the query tiles of one
  // (head, key range) are consecutive and share an XCD.
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % ntq, hp = logical / ntq;
  const int bh = SPLIT ? hp / nsplit : hp, part = SPLIT ? hp - bh * nsplit : 0;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint32_t hbytes = (uint32_t)N * D * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes);
  const rsrc_t rk = make_rsrc(k + hoff, hbytes);
  const rsrc_t rv = make_rsrc(v + hoff, hbytes);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, g = lane >> 5;
  // query rows of this lane: qrow0 + 32*qb, qb = 0..QB-1
  const int qrow0 = qt * C::BR + wave * 32 * QB + li;

  // Q^T as B operands, held for the whole loop: k-step kk covers columns
  // kk*16 + 8g .. +7 of this lane's query rows.
  bf16x8 qreg[QB][C::DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk)
      qreg[qb][kk] = as_bf16x8(
          buf_load16(rq, (uint32_t)(((qrow0 + 32 * qb) * D + kk * 16 + g * 8) * 2)));

  f32x16 acc[QB][C::DB];   // O^T blocks: rows = columns of O, col = this lane's query
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[qb][db] = zero16();
  // Reference value (log2 units) and this lane's share of l; lb is the same
  // sum taken over the bf16-rounded P~ that the PV contraction multiplies.
  float m_run[QB], l_run[QB], lb_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
    lb_run[qb] = 0.0f;
  }

  // Key tiles [j0, j1): all of them, or this workgroup's range in split mode
  // (whole tiles, as even as possible; every range holds at least one tile).
  const int nkt = (N + BC - 1) / BC;
  const int j0 = SPLIT ? (int)((int64_t)part * nkt / nsplit) : 0;
  const int j1 = SPLIT ? (int)((int64_t)(part + 1) * nkt / nsplit) : nkt;
  // K and V tiles in row-segment order (K swizzled for its row-operand
  // reads, V plain for its transposing reads); buffer b at byte
  // b * BUF_ELEMS * 2, K then V.
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t kvoff = seg_dma_voff<D, C::WAVES, true>(wave, lane);
  const uint32_t vvoff = seg_dma_voff<D, C::WAVES, false>(wave, lane);
  constexpr int NU = (BC / 16) * (D / 32) / C::WAVES;   // loads per tile and wave
  static_assert(NU * C::WAVES == (BC / 16) * (D / 32), "whole loads per wave");
  auto load_tile = [&](int jt, int b) {
    uint32_t kd = lds0 + (uint32_t)(b * C::BUF_ELEMS * 2), vd = kd + (uint32_t)(C::TILE * 2);
    const uint32_t r0 = (uint32_t)(jt * BC * D * 2);
    asm volatile("" : "+s"(kd), "+s"(vd));   // one address per buffer, not one per load
#pragma unroll
    for (int u = 0; u < NU; ++u) seg_dma<D, C::WAVES>(kd, rk, kvoff, r0, wave, u);
#pragma unroll
    for (int u = 0; u < NU; ++u) seg_dma<D, C::WAVES>(vd, rv, vvoff, r0, wave, u);
  };
  const uint32_t kbase0 = seg_rowop_base<D>(lane, 0), kbase1 = seg_rowop_base<D>(lane, 1);
  const uint32_t vbase = seg_trop_base<D>(lane);
  load_tile(j0, 0);
  wait_vmem();
  __syncthreads();

  for (int j = j0; j < j1; ++j) {
    const int jb = (j - j0) & 1;   // buffer of tile j
    uint32_t bo = (uint32_t)(jb * C::BUF_ELEMS * 2);
    asm volatile("" : "+s"(bo));
    const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(smem) + bo;
    const uint8_t* kl[2] = {kb8 + kbase0, kb8 + kbase1};   // this lane's K reads
    const uint8_t* vl = kb8 + C::TILE * 2 + vbase;          // ... and V reads
    auto kread = [&](int kb, int kk) {
      return *reinterpret_cast<const bf16x8*>(kl[kk & 1] + seg_rowop_imm<D>(kb, kk));
    };
    if (j + 1 < j1) load_tile(j + 1, jb ^ 1);

    // S^T = K_j Q^T in 32-key blocks; A = K rows from LDS (each read feeds
    // the QB query blocks), B = Q^T.  The K operands are read kReadAhead
    // k-steps ahead of the instructions that use them (a scheduling fence
    // keeps the compiler from sinking the reads next to their uses, which
    // would expose the LDS latency once per instruction), and the key blocks
    // alternate so that consecutive matrix-core instructions are independent.
    constexpr int RA = kReadAhead;
    f32x16 s[QB][C::KB];
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    bf16x8 kop[RA + 1][C::KB];
#pragma unroll
    for (int kk = 0; kk < RA; ++kk)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) kop[kk][kb] = kread(kb, kk);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = zero16();
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk) {
      if (kk + RA < C::DK) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
          kop[(kk + RA) % (RA + 1)][kb] = kread(kb, kk + RA);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = mfma32(kop[kk % (RA + 1)][kb], qreg[qb][kk], s[qb][kb]);
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
    // Keys past N in the last tile do not exist: their scores are -inf.
    if (j * BC + BC > N) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j * BC + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key >= N) s[qb][kb][i] = -INFINITY;
          }
    }

    // Online softmax for each of this lane's query rows.  The reference
    // value m_run moves only when some row of the wave sees a score more
    // than 2^kSlack above it; until then the factor 2^(m_old - m_new) would
    // be 1 for the rows that did not grow and the rescale is skipped.
    // P~ = 2^(c s - m_run) then stays <= 2^kSlack, and because U and l share
    // the same reference value the result O = U / l is unchanged (the
    // rescale identity holds for any common reference, not only the maximum).
    // No row maximum is taken on the common path: the exponentials are
    // formed against the current reference first, and their fp32 lane sum
    // tells whether it has to move.
    bf16x8 pb[QB][BC / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Exponentials against the current reference, packed to bf16; rs is
      // this lane's fp32 sum, rb the sum of the packed values.
      float rs, rb;
      auto exps = [&]() {
        float r = 0.0f, b0 = 0.0f, b1 = 0.0f;
#pragma unroll
        for (int t = 0; t < BC / 16; ++t) {
          const int kb = t >> 1, h = t & 1;
          u32x4 pw;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(s[qb][kb][8 * h + 2 * e], c2, -m_run[qb]));
            const float p1 = fast_exp2(fmaf(s[qb][kb][8 * h + 2 * e + 1], c2, -m_run[qb]));
            r += p0 + p1;
            pw[e] = pack_bf16x2(p0, p1);
            if (e & 1) b1 = add_bf16x2(pw[e], b1);
            else b0 = add_bf16x2(pw[e], b0);
          }
          pb[qb][t] = as_bf16x8(pw);
        }
        rs = r;
        rb = b0 + b1;
      };
      exps();
      // The reference must move when some P~ exceeds 2^kSlack; a lane sum
      // above that (or not a number: first tile, m_run = -inf) is necessary
      // for it, and only then is the row maximum taken.
      if (__any(!(rs <= kSlackPow))) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb][i]);
        mx = max_across_halves(mx);
        const float m_new = fmaxf(m_run[qb], mx * c2);
        const float alpha = fast_exp2(m_run[qb] - m_new);   // 0 on the first tile
        l_run[qb] *= alpha;
        lb_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha;
        m_run[qb] = m_new;
        exps();
      }
      l_run[qb] += rs;
      lb_run[qb] += rb;
    }

    // O^T += V_j^T P^T over steps n = (t, db): 16-key step t, 32-column
    // block db.  The V^T operand of a step is gathered with transposing
    // reads kStepAhead steps ahead (behind a scheduling fence) and feeds the
    // QB query blocks.
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    {
      constexpr int SA = kStepAhead, NS = (BC / 16) * C::DB;
      bf16x8 vop[SA + 1];
#pragma unroll
      for (int n = 0; n < SA; ++n) vop[n] = seg_trop_read<D>(vl, n / C::DB, n % C::DB);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + SA < NS) {
          const int m = n + SA;
          vop[m % (SA + 1)] = seg_trop_read<D>(vl, m / C::DB, m % C::DB);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int t = n / C::DB, db = n % C::DB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32(vop[n % (SA + 1)], pb[qb][t], acc[qb][db]);
      }
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);

    wait_vmem();      // this wave's loads of tile j+1 have landed in LDS
    __syncthreads();  // ... and everyone's; tile j is no longer read
  }

  // Epilogue: O = U / l, LSE = ln2 * (m + log2 l).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qrow0 + 32 * qb;
    // O is divided by the sum of the rounded weights it was accumulated
    // with, so it is a convex combination of V rows whatever the rounding
    // (a dominant key's rounding cancels); the LSE uses the fp32 sum.
    const float l_tot = sum_across_halves(l_run[qb]);
    const float lb_tot = sum_across_halves(lb_run[qb]);
    if (qrow < N) {
      const float inv = 1.0f / lb_tot;
      if (SPLIT) {   // fp32 output of this key range, at part p of the partial tensors
        float* orow = static_cast<float*>(o) + part * part_rows * D + hoff + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc[qb][db][4 * r + e] * inv;
            *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * r + 4 * g) = w;
          }
      } else {
        uint16_t* orow = static_cast<uint16_t*>(o) + hoff + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[qb][db][4 * r + 0] * inv, acc[qb][db][4 * r + 1] * inv);
            w[1] = pack_bf16x2(acc[qb][db][4 * r + 2] * inv, acc[qb][db][4 * r + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * r + 4 * g) = w;
          }
      }
      if (g == 0)
        lse[(SPLIT ? part * part_rows : 0) + (int64_t)bh * N + qrow] =
            kLn2 * (m_run[qb] + log2f(l_tot));
    }
  }
}

template <int D, int QB, int BC, int MINW, bool PRIO, int NWAVES = 4, bool SPLIT = false>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, float* lse,
           int64_t BH, int64_t N, float scale, int nsplit, hipStream_t stream) {
  using C = FwdCfg<D, QB, BC, NWAVES>;
  const int ntq = (int)((N + C::BR - 1) / C::BR);
  const int64_t nwg = (int64_t)ntq * BH * nsplit;
  auto kern = fwd_bf16_kernel<D, QB, BC, MINW, PRIO, NWAVES, SPLIT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(C::THREADS), C::LDS_BYTES, stream, q, k,
                     v, o, lse, (int)N, ntq, scale * kLog2e, nsplit, BH * N);
  return (int)hipGetLastError();
}

}  // namespace

int launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream) {
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  auto* o16 = static_cast<uint16_t*>(o);
  // d = 128: 8 waves x 32 query rows, key tiles of 128 (one workgroup per CU,
  // two waves per SIMD); d = 64: 8 waves x 32 rows, key tiles of 64 (two
  // workgroups per CU).
  if (d == 128)
    return launch<128, 1, 128, 2, true, 8>(q16, k16, v16, o16, lse, BH, N, scale, 1, stream);
  return launch<64, 1, 64, 2, false, 8>(q16, k16, v16, o16, lse, BH, N, scale, 1, stream);
}

int fwd_split_tile(int64_t d) { return d == 128 ? 128 : 64; }

int launch_fwd_split_bf16(const void* q, const void* k, const void* v, float* o_part,
                          float* lse_part, int64_t BH, int64_t N, int64_t d, float scale,
                          int nsplit, hipStream_t stream) {
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  if (d == 128)
    return launch<128, 1, 128, 2, true, 8, true>(q16, k16, v16, o_part, lse_part, BH, N, scale,
                                                 nsplit, stream);
  return launch<64, 1, 64, 2, false, 8, true>(q16, k16, v16, o_part, lse_part, BH, N, scale,
                                              nsplit, stream);
}

}  // namespace fa
