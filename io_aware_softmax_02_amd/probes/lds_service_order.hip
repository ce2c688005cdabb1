// LDS bank-conflict probe for 16-byte reads (ds_read_b128) and 8-byte
// transposing reads (ds_read_b64_tr_b16) on gfx950.  Not part of the
// library: a standalone program whose dispatches are read with rocprofv3
// counters (SQ_LDS_BANK_CONFLICT, SQ_INSTS_LDS, SQ_LDS_IDX_ACTIVE), one
// kernel instantiation per lane->address pattern.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       io_aware_softmax_02_amd/probes/lds_service_order.hip -o /tmp/lds_service_order
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE -f csv \
//       -d OUT -o p -- /tmp/lds_service_order
//
// Each wave reads a fixed per-lane byte offset (a table, checked on the host
// to lie inside the 16 KB buffer and to be aligned) ITERS times.  The
// patterns are the attention kernels' own row-operand and transposing reads
// (with the row-segment swizzles used before and the one used now) and
// synthetic permutations that identify which lanes a 16-byte read serves
// together.  The program prints the pattern index -> name table; the
// dispatch of pattern i is the kernel probe<kind, i>.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
constexpr int LDS = 16384, ITERS = 4096, BLOCKS = 1024;

template <int KIND, int PAT>   // KIND 0: ds_read_b128, 1: ds_read_b64_tr_b16
__global__ __launch_bounds__(64) void probe(const uint32_t* __restrict__ offs,
                                            uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t sm[LDS / 4];
  const int lane = threadIdx.x;
  for (int i = lane; i < LDS / 4; i += 64) sm[i] = i * 2654435761u;
  __syncthreads();
  uint32_t off = offs[lane];
  uint32_t acc = 0;
  for (int it = 0; it < ITERS; ++it) {
    asm volatile("" : "+v"(off));   // opaque address: one read per iteration
    const __attribute__((address_space(3))) char* base =
        (const __attribute__((address_space(3))) char*)sm + off;
    if (KIND == 0) {
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base);
      acc += v[0] ^ v[1] ^ v[2] ^ v[3];
    } else {
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(base));
      acc += (uint32_t)(uint16_t)v[0] ^ (uint32_t)(uint16_t)v[3];
    }
    asm volatile("" : "+v"(acc));
  }
  out[blockIdx.x * 64 + lane] = acc;
}

// Piece swizzles of a 64-byte row segment (four 16-byte pieces), by row rho
// of a 16-row block: the two used before (for row reads; for row and
// transposing reads) and the current one.
static int swz_rows_old(int rho) { return (rho >> 2) & 3; }
static int swz_both_old(int rho) { return 2 * ((rho >> 2) & 1) + ((rho >> 3) & 1); }
static int swz_now(int rho) { return 2 * ((rho >> 2) & 1); }

struct Pattern {
  std::string name;
  int kind;
  std::vector<uint32_t> off;
};

template <typename F>
static Pattern make(const char* name, int kind, F f) {
  Pattern p{name, kind, {}};
  for (int l = 0; l < 64; ++l) p.off.push_back((uint32_t)f(l));
  return p;
}

// Row operand of the 16 x 16 x 32 instruction: lane l reads row l % 16,
// piece l / 16.  Transposing read: source lane 4a + b of group g addresses
// row 4g + a, bytes 16 ((2e + (b >> 1)) ^ swz) + 8 (b & 1).
template <typename S>
static int rowop(int l, S swz) { return 64 * (l & 15) + 16 * ((l >> 4) ^ swz(l & 15)); }
template <typename S>
static int trop(int l, S swz) {
  const int i16 = l & 15, g = l >> 4, a = i16 >> 2, b = i16 & 3, rho = 4 * g + a;
  return 64 * rho + 16 * ((b >> 1) ^ swz(rho)) + 8 * (b & 1);
}

int main() {
  std::vector<Pattern> ps;
  ps.push_back(make("linear 16 B per lane", 0, [](int l) { return 16 * l; }));
  ps.push_back(make("row operand, no swizzle", 0, [](int l) { return rowop(l, [](int) { return 0; }); }));
  ps.push_back(make("row operand, old row swizzle", 0, [](int l) { return rowop(l, swz_rows_old); }));
  ps.push_back(make("row operand, old both swizzle", 0, [](int l) { return rowop(l, swz_both_old); }));
  ps.push_back(make("row operand, current swizzle", 0, [](int l) { return rowop(l, swz_now); }));
  ps.push_back(make("quarter-waves swapped (l^16)", 0, [](int l) { return 16 * (l ^ 16); }));
  ps.push_back(make("quarter-waves rotated by 4q", 0,
                    [](int l) { return 16 * (16 * (l >> 4) + (((l & 15) + 4 * (l >> 4)) & 15)); }));
  ps.push_back(make("transpose 8x8", 0, [](int l) { return 16 * (8 * (l & 7) + (l >> 3)); }));
  ps.push_back(make("stride 32 B", 0, [](int l) { return 32 * l; }));
  ps.push_back(make("stride 64 B", 0, [](int l) { return 64 * l; }));
  ps.push_back(make("transposing read, old both swizzle", 1, [](int l) { return trop(l, swz_both_old); }));
  ps.push_back(make("transposing read, current swizzle", 1, [](int l) { return trop(l, swz_now); }));
  for (const auto& p : ps)
    for (auto o : p.off)
      if (o + 16 > (uint32_t)LDS || o % (p.kind == 0 ? 16 : 8)) {
        std::printf("offset %u of pattern '%s' outside the buffer or misaligned\n", o, p.name.c_str());
        return 1;
      }
  uint32_t *doff = nullptr, *dout = nullptr;
  if (hipMalloc(&doff, 64 * 4) != hipSuccess || hipMalloc(&dout, BLOCKS * 64 * 4) != hipSuccess) {
    std::printf("hipMalloc failed\n");
    return 1;
  }
  for (size_t i = 0; i < ps.size(); ++i) {
    const Pattern& p = ps[i];
    if (hipMemcpy(doff, p.off.data(), 64 * 4, hipMemcpyHostToDevice) != hipSuccess) return 1;
    switch (i) {
#define CASE(n)                                                                                  \
  case n:                                                                                        \
    if (p.kind == 0)                                                                             \
      hipLaunchKernelGGL((probe<0, n>), dim3(BLOCKS), dim3(64), 0, 0, doff, dout);               \
    else                                                                                         \
      hipLaunchKernelGGL((probe<1, n>), dim3(BLOCKS), dim3(64), 0, 0, doff, dout);               \
    break;
      CASE(0) CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10)
      CASE(11)
#undef CASE
      default: return 1;
    }
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    std::printf("pattern %2zu: %s\n", i, p.name.c_str());
  }
  const hipError_t e = hipGetLastError();
  std::printf("status %s\n", hipGetErrorString(e));
  return e != hipSuccess;
}
