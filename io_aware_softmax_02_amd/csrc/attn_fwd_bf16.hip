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
//   workgroup = NWAVES waves; each wave owns two 16-row blocks of query rows
//   of one (batch, head).  Key tiles of BC rows stream through LDS,
//   double-buffered: direct buffer->LDS loads of tile j+1 are issued at the
//   start of tile j (no registers involved), one barrier per tile.
//   Both contractions use the 16 x 16 x 32 matrix-core instruction
//   (device_common.h), which sustains a higher rate than the 32 x 32 x 16
//   form on data of unit scale; every K or V operand read from LDS feeds the
//   two query blocks.
//   Scores are formed transposed, S^T = K Q^T, so that a lane owns query
//   rows: lane l holds query l%16 of each block for keys 4(l/16) + 0..3 of
//   every 16 keys, so a row's keys are spread over the four lanes l, l^16,
//   l^32, l^48.  Row sums are in-lane (combined across the four at the end);
//   the row max, taken only when the softmax reference has to move, is an
//   in-lane reduction plus two lane exchanges.  Two 16-key score
//   accumulators, converted to bf16, are already the 32-key B operand of one
//   O^T += V^T P^T step, so P never touches LDS; the V^T operand is gathered
//   from the V tile with transposing LDS reads in the matching key order.
//   Both tiles are stored in row-segment order (lds_tile.h): every direct
//   load reads whole 64-byte row segments, the rate at which the load path
//   runs at full speed, and every LDS read is a base register (two for V)
//   plus an immediate offset, free of bank conflicts.
//   Base-2 domain: c = scale * log2(e); p = 2^(c s - m) with m in log2 units;
//   LSE = ln 2 * (m + log2 l).
//
// Split-KV mode (SPLIT): the key tiles are cut into nsplit contiguous ranges
// and each workgroup handles one range of one query tile, writing that
// range's own normalised output (fp32) and LSE.  The ranges are recombined
// by the merge kernel (attn_merge.hip) with the same rescale identity.
#include "launch_chunks.h"
#include "lds_tile.h"

namespace fa {
namespace {

// Slack of the lazily updated softmax reference, in log2 units.
constexpr float kSlack = 8.0f;
constexpr float kSlackPow = 256.0f;   // 2^kSlack

template <int D, int BC, int NWAVES>
struct FwdCfg {
  static constexpr int WAVES = NWAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = WAVES * 32;           // query rows per workgroup
  static constexpr int KB = BC / 16;              // 16-key score blocks per tile
  static constexpr int NT = BC / 32;              // 32-key steps of the PV contraction
  static constexpr int TILE = BC * D;             // one K or V tile (bf16)
  static constexpr int BUF_ELEMS = 2 * TILE;      // K tile then V tile
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int DK = D / 32;               // k-steps of the QK^T contraction
  static constexpr int DB = D / 16;               // 16-column blocks of O
  static_assert(BC % 32 == 0 && BC <= 128, "key tile is a multiple of 32 rows");
};

// K operands (counted in operands) and V^T operands (in (t, db) steps) are
// read from LDS this far ahead of the instructions that use them, behind a
// scheduling fence that keeps the compiler from sinking each read next to
// its use (which would expose the LDS latency once per instruction).
constexpr int kReadAhead = 4;
constexpr int kStepAhead = 6;

template <int D, int BC, int MINW, bool PRIO, int NWAVES, bool SPLIT, int RA = kReadAhead,
          int SA = kStepAhead>
__global__ __launch_bounds__(64 * NWAVES, MINW) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, void* __restrict__ o, float* __restrict__ lse, int N,
    int ntq, float c2, int nsplit, int64_t part_rows) {
  using C = FwdCfg<D, BC, NWAVES>;
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
  const int li = lane & 15, g = lane >> 4;
  // query rows of this lane: qrow0 (block 0) and qrow0 + 16 (block 1)
  const int qrow0 = qt * C::BR + wave * 32 + li;

  // Q^T as B operands: k-step kk covers columns 32 kk + 8 g .. +7.
  bf16x8 qreg[2][C::DK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk)
      qreg[qb][kk] = as_bf16x8(
          buf_load16(rq, (uint32_t)(((qrow0 + 16 * qb) * D + kk * 32 + g * 8) * 2)));

  // O^T blocks: lane l holds columns 16 db + 4 g + 0..3 of its query.
  f32x4 acc[2][C::DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[2], l_run[2], lb_run[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
    lb_run[qb] = 0.0f;
  }

  // Key tiles [j0, j1): all of them, or this workgroup's range in split mode
  // (whole tiles, as even as possible; every range holds at least one tile).
  const int nkt = (N + BC - 1) / BC;
  const int j0 = SPLIT ? (int)((int64_t)part * nkt / nsplit) : 0;
  const int j1 = SPLIT ? (int)((int64_t)(part + 1) * nkt / nsplit) : nkt;
  // K and V tiles in row-segment order (lds_tile.h), whose swizzle keeps
  // both K's row-operand reads and V's transposing reads free of bank
  // conflicts; buffer b at byte b * BUF_ELEMS * 2, K then V.
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t voff = seg_dma_voff<D, C::WAVES>(wave, lane);
  constexpr int NU = (BC / 16) * (D / 32) / C::WAVES;
  static_assert(NU * C::WAVES == (BC / 16) * (D / 32), "whole loads per wave");
  auto load_tile = [&](int jt, int b) {
    uint32_t kd = lds0 + (uint32_t)(b * C::BUF_ELEMS * 2), vd = kd + (uint32_t)(C::TILE * 2);
    const uint32_t r0 = (uint32_t)(jt * BC * D * 2);
    asm volatile("" : "+s"(kd), "+s"(vd));   // one address per buffer, not one per load
#pragma unroll
    for (int u = 0; u < NU; ++u) seg_dma<D, C::WAVES>(kd, rk, voff, r0, wave, u);
#pragma unroll
    for (int u = 0; u < NU; ++u) seg_dma<D, C::WAVES>(vd, rv, voff, r0, wave, u);
  };
  const uint32_t kbase = seg_rowop16_base(lane);
  const uint32_t vbase0 = seg_trop16_base(lane, 0), vbase1 = seg_trop16_base(lane, 1);
  load_tile(j0, 0);
  wait_vmem();
  __syncthreads();

  for (int j = j0; j < j1; ++j) {
    const int jb = (j - j0) & 1;
    uint32_t bo = (uint32_t)(jb * C::BUF_ELEMS * 2);
    asm volatile("" : "+s"(bo));
    const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(smem) + bo;
    const uint8_t* kl = kb8 + kbase;
    const uint8_t* vl[2] = {kb8 + C::TILE * 2 + vbase0, kb8 + C::TILE * 2 + vbase1};
    auto kread = [&](int n) {
      return *reinterpret_cast<const bf16x8*>(kl + seg_rowop16_imm<D>(n % C::KB, n / C::KB));
    };
    auto vread = [&](int n) {
      const int db = n % C::DB;
      return seg_trop16_read<D>(vl[db & 1], n / C::DB, db);
    };
    if (j + 1 < j1) load_tile(j + 1, jb ^ 1);

    // S^T = K_j Q^T: operand n is (key block n % KB, k-step n / KB) and
    // feeds both query blocks; an accumulator is reused KB operands later.
    f32x4 s[2][C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[qb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    {
      constexpr int NS = C::DK * C::KB;
      bf16x8 kop[RA + 1];
#pragma unroll
      for (int n = 0; n < RA; ++n) kop[n] = kread(n);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + RA < NS) kop[(n + RA) % (RA + 1)] = kread(n + RA);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = n % C::KB, kk = n / C::KB;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[qb][kb] = mfma16(kop[n % (RA + 1)], qreg[qb][kk], s[qb][kb]);
      }
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
    // Keys past N in the last tile do not exist: their scores are -inf.
    if (j * BC + BC > N) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (j * BC + kb * 16 + 4 * g + i >= N) s[qb][kb][i] = -INFINITY;
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
    bf16x8 pb[2][C::NT];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // Exponentials against the current reference, packed to bf16 in the
      // B-operand order of the PV step; rs is this lane's fp32 sum, rb the
      // sum of the packed values.
      float rs, rb;
      auto exps = [&]() {
        float r = 0.0f, b0 = 0.0f, b1 = 0.0f;
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
          u32x4 pw;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kb = 2 * t + (e >> 1), i = 2 * (e & 1);
            const float p0 = fast_exp2(fmaf(s[qb][kb][i], c2, -m_run[qb]));
            const float p1 = fast_exp2(fmaf(s[qb][kb][i + 1], c2, -m_run[qb]));
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
      // for it, and only then is the row maximum taken (over the four lanes
      // that share the row).
      if (__any(!(rs <= kSlackPow))) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
        mx = max_across_quarters(mx);
        const float m_new = fmaxf(m_run[qb], mx * c2);
        const float alpha = fast_exp2(m_run[qb] - m_new);   // 0 on the first tile
        l_run[qb] *= alpha;
        lb_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[qb][db][i] *= alpha;
        m_run[qb] = m_new;
        exps();
      }
      l_run[qb] += rs;
      lb_run[qb] += rb;
    }

    // O^T += V_j^T P^T over steps n = (t, db); each V^T operand feeds both
    // query blocks, and an accumulator is reused DB steps later.
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    {
      constexpr int NS = C::NT * C::DB;
      bf16x8 vop[SA + 1];
#pragma unroll
      for (int n = 0; n < SA; ++n) vop[n] = vread(n);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        if (n + SA < NS) vop[(n + SA) % (SA + 1)] = vread(n + SA);
        __builtin_amdgcn_sched_barrier(0);
        const int t = n / C::DB, db = n % C::DB;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc[qb][db] = mfma16(vop[n % (SA + 1)], pb[qb][t], acc[qb][db]);
      }
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);

    wait_vmem();      // this wave's loads of tile j+1 have landed in LDS
    __syncthreads();  // ... and everyone's; tile j is no longer read
  }

  // Epilogue: O = U / l, LSE = ln2 * (m + log2 l).  O is divided by the sum
  // of the rounded weights it was accumulated with, so it is a convex
  // combination of V rows whatever the rounding (a dominant key's rounding
  // cancels); the LSE uses the fp32 sum.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qrow0 + 16 * qb;
    const float l_tot = sum_across_quarters(l_run[qb]);
    const float lb_tot = sum_across_quarters(lb_run[qb]);
    if (qrow < N) {
      const float inv = 1.0f / lb_tot;
      if (SPLIT) {   // fp32 output of this key range, at part p of the partial tensors
        float* orow = static_cast<float*>(o) + part * part_rows * D + hoff + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          f32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = acc[qb][db][i] * inv;
          *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g) = w;
        }
      } else {
        uint16_t* orow = static_cast<uint16_t*>(o) + hoff + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[qb][db][0] * inv, acc[qb][db][1] * inv);
          w[1] = pack_bf16x2(acc[qb][db][2] * inv, acc[qb][db][3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * g) = w;
        }
      }
      if (g == 0)
        lse[(SPLIT ? part * part_rows : 0) + (int64_t)bh * N + qrow] =
            kLn2 * (m_run[qb] + log2f(l_tot));
    }
  }
}

template <int D, int BC, int MINW, bool PRIO, int NWAVES, bool SPLIT = false,
          int RA = kReadAhead, int SA = kStepAhead>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, float* lse,
             int64_t BH, int64_t N, float scale, int nsplit, hipStream_t stream) {
  using C = FwdCfg<D, BC, NWAVES>;
  const int ntq = (int)((N + C::BR - 1) / C::BR);
  const int64_t per_head = (int64_t)ntq * nsplit * C::THREADS;
  if (!unit_fits(per_head)) return kErrGridTooLarge;
  auto kern = fwd_bf16_kernel<D, BC, MINW, PRIO, NWAVES, SPLIT, RA, SA>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  // Chunks of whole heads; the partials keep their stride of B*H*N rows.
  return launch_in_chunks(BH, per_head, [&](int64_t h0, int64_t nh) {
    const int64_t off = h0 * N * D;
    void* oc = SPLIT ? (void*)(static_cast<float*>(o) + off)
                     : (void*)(static_cast<uint16_t*>(o) + off);
    hipLaunchKernelGGL(kern, dim3((unsigned)(ntq * nh * nsplit)), dim3(C::THREADS),
                       C::LDS_BYTES, stream, q + off, k + off, v + off, oc, lse + h0 * N, (int)N,
                       ntq, scale * kLog2e, nsplit, BH * N);
    return (int)hipGetLastError();
  });
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
    return launch<128, 128, 2, true, 8>(q16, k16, v16, o16, lse, BH, N, scale, 1, stream);
  return launch<64, 64, 2, true, 8>(q16, k16, v16, o16, lse, BH, N, scale, 1, stream);
}

int fwd_split_tile(int64_t d) { return d == 128 ? 128 : 64; }

int launch_fwd_split_bf16(const void* q, const void* k, const void* v, float* o_part,
                          float* lse_part, int64_t BH, int64_t N, int64_t d, float scale,
                          int nsplit, hipStream_t stream) {
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  if (d == 128)
    return launch<128, 128, 2, true, 8, true>(q16, k16, v16, o_part, lse_part, BH, N, scale,
                                              nsplit, stream);
  return launch<64, 64, 2, true, 8, true>(q16, k16, v16, o_part, lse_part, BH, N, scale, nsplit,
                                          stream);
}

}  // namespace fa
