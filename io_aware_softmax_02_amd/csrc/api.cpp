// C ABI entry points declared in include/fa.h: argument checks (validate.h),
// then launches on the caller's stream.  Nothing is allocated here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"
#include "launch_chunks.h"
#include "validate.h"

// Scratch of fa_bwd_noalloc: D = rowsum(dO * O), one fp32 per query row, for
// at most FA_BWD_NOALLOC_MAX_ROWS rows (16 MiB).  Every GPU the library runs
// on holds its own copy from the time the code object is loaded until the
// process ends.  In host code this name is only a handle for
// hipGetSymbolAddress: the device address comes from that call, per device.
static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace fa {
int launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream);
int launch_bwd_pre_bf16(const void* o, const void* dO, float* delta, int64_t rows, int64_t d,
                        hipStream_t stream);
int launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const float* lse,
                         const void* dO, const float* delta, void* dk, void* dv, int64_t BH,
                         int64_t N, int64_t d, float scale, hipStream_t stream);
int launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const float* lse,
                       const void* dO, const float* delta, void* dq, int64_t BH, int64_t N,
                       int64_t d, float scale, hipStream_t stream);
int fwd_split_tile(int64_t d);
int launch_fwd_split_bf16(const void* q, const void* k, const void* v, float* o_part,
                          float* lse_part, int64_t BH, int64_t N, int64_t d, float scale,
                          int nsplit, hipStream_t stream);
int launch_merge_bf16(const float* o_part, const float* lse_part, int nsplit, int64_t rows,
                      int64_t d, void* o, float* lse, hipStream_t stream);
int f32_key_block(int64_t N, int64_t d);
int launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int64_t BH, int64_t N, int64_t d, float scale, hipStream_t stream);
int launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                   const float* lse, const float* dO, float* dq, float* dk, float* dv,
                   float* delta, int64_t BH, int64_t N, int64_t d, float scale,
                   hipStream_t stream);
}  // namespace fa

namespace {

using fa::Shape;
using fa::Span;

// Launcher status: 0, a hipError_t, or kErrGridTooLarge (one head's grid
// exceeds a launch; reported before anything is enqueued).
inline fa_status from_hip(int e) {
  if (e == 0) return FA_OK;
  return e == fa::kErrGridTooLarge ? FA_ERR_SHAPE : FA_ERR_HIP;
}
inline hipStream_t as_stream(fa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

struct Sizes {
  size_t tensor, rows;
};
inline Sizes sizes(const Shape& s, size_t elem) {
  return {static_cast<size_t>(s.elems()) * elem, static_cast<size_t>(s.rows()) * sizeof(float)};
}

fa_status check_fwd(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const Shape& s, float scale, bool bf16) {
  FA_TRY(fa::check_shape(s, bf16));
  FA_TRY(fa::check_scale(scale));
  if (s.empty()) return FA_OK;
  const size_t al = bf16 ? 16 : 4;
  FA_TRY(fa::check_ptrs({q, k, v, o}, al));
  FA_TRY(fa::check_ptrs({lse}, bf16 ? 16 : 4));
  const Sizes z = sizes(s, bf16 ? 2 : 4);
  return fa::check_alias({{q, z.tensor}, {k, z.tensor}, {v, z.tensor}},
                         {{o, z.tensor}, {lse, z.rows}});
}

fa_status check_bwd(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, const void* dq, const void* dk,
                    const void* dv, const void* ws, size_t ws_bytes, const Shape& s,
                    float scale, bool bf16) {
  FA_TRY(fa::check_shape(s, bf16));
  FA_TRY(fa::check_scale(scale));
  if (s.empty()) return FA_OK;
  const size_t al = bf16 ? 16 : 4;
  FA_TRY(fa::check_ptrs({q, k, v, o, dO, dq, dk, dv}, al));
  FA_TRY(fa::check_ptrs({lse}, bf16 ? 16 : 4));
  FA_TRY(fa::check_workspace(ws, ws_bytes, fa::bwd_workspace_bytes(s, bf16)));
  const Sizes z = sizes(s, bf16 ? 2 : 4);
  const size_t wsz = fa::bwd_workspace_bytes(s, bf16);
  return fa::check_alias({{q, z.tensor}, {k, z.tensor}, {v, z.tensor}, {o, z.tensor},
                          {lse, z.rows}, {dO, z.tensor}},
                         {{dq, z.tensor}, {dk, z.tensor}, {dv, z.tensor}, {ws, wsz}});
}

// A call's kernels run on its stream's device, while kernel attributes (the
// dynamic LDS size) are set on the current device.  For a stream of another
// device, that device is made current for the call and the caller's device
// is restored afterwards; the null stream is the current device's.  A stream
// whose device cannot be read is left to the launch to report.
class OnStreamDevice {
 public:
  explicit OnStreamDevice(hipStream_t st) {
    int dev = -1;
    if (st == nullptr || hipStreamGetDevice(st, &dev) != hipSuccess) return;
    if (hipGetDevice(&prev_) != hipSuccess) return;
    if (dev != prev_) {
      ok_ = hipSetDevice(dev) == hipSuccess;
      switched_ = ok_;
    }
  }
  ~OnStreamDevice() {
    if (switched_) (void)hipSetDevice(prev_);
  }
  OnStreamDevice(const OnStreamDevice&) = delete;
  OnStreamDevice& operator=(const OnStreamDevice&) = delete;
  bool ok() const { return ok_; }

 private:
  int prev_ = -1;
  bool ok_ = true, switched_ = false;
};

#define FA_ON_STREAM_DEVICE(st)                   \
  const OnStreamDevice fa_on_device_(st);         \
  if (!fa_on_device_.ok()) return FA_ERR_HIP

// Device address of `scratch` on device `dev`, looked up once per device
// with that device current (each device holds the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fa_status scratch_on(int dev, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return FA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative size or size too large";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim not supported (bf16: 64 or 128; fp32: 1..128)";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointer not aligned (bf16 path: 16 bytes; fp32 path: 4 bytes)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace smaller than required";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or another output";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a launch";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: B*H*N exceeds the fixed scratch of fa_bwd_noalloc (FA_BWD_NOALLOC_MAX_ROWS rows)";
  }
  return "unknown fa_status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                 int64_t H, int64_t N, int64_t d, float scale, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_fwd(q, k, v, o, lse, s, scale, true));
  if (s.empty()) return FA_OK;
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, scale, as_stream(stream)));
}

int64_t fa_fwd_split_max(int64_t B, int64_t H, int64_t N, int64_t d) {
  const Shape s{B, H, N, d};
  if (fa::check_shape(s, true) != FA_OK) return -1;
  return fa::split_max(s, fa::fwd_split_tile(d));
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, float* o_part,
                       float* lse_part, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       int64_t n_split, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(fa::check_shape(s, true));
  FA_TRY(fa::check_scale(scale));
  FA_TRY(fa::check_parts(s, n_split));
  if (s.empty()) return FA_OK;
  if (n_split > fa::split_max(s, fa::fwd_split_tile(d))) return FA_ERR_SHAPE;
  FA_TRY(fa::check_ptrs({q, k, v, o_part, lse_part}, 16));
  const Sizes z = sizes(s, 2);
  const size_t np = static_cast<size_t>(n_split);
  FA_TRY(fa::check_alias({{q, z.tensor}, {k, z.tensor}, {v, z.tensor}},
                         {{o_part, np * z.tensor * 2}, {lse_part, np * z.rows}}));
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_fwd_split_bf16(q, k, v, o_part, lse_part, B * H, N, d, scale,
                                            static_cast<int>(n_split), as_stream(stream)));
}

fa_status fa_merge(const float* o_part, const float* lse_part, int64_t n_split, void* o,
                   float* lse, int64_t B, int64_t H, int64_t N, int64_t d, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(fa::check_shape(s, true));
  FA_TRY(fa::check_parts(s, n_split));
  if (s.empty()) return FA_OK;
  FA_TRY(fa::check_ptrs({o_part, lse_part, o, lse}, 16));
  const Sizes z = sizes(s, 2);
  const size_t np = static_cast<size_t>(n_split);
  FA_TRY(fa::check_alias({{o_part, np * z.tensor * 2}, {lse_part, np * z.rows}},
                         {{o, z.tensor}, {lse, z.rows}}));
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_merge_bf16(o_part, lse_part, static_cast<int>(n_split), s.rows(),
                                        d, o, lse, as_stream(stream)));
}

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return fa::bwd_workspace_bytes(Shape{B, H, N, d}, true);
}

fa_status fa_bwd_preprocess(const void* o, const void* dO, float* delta, int64_t B, int64_t H,
                            int64_t N, int64_t d, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(fa::check_shape(s, true));
  if (s.empty()) return FA_OK;
  FA_TRY(fa::check_ptrs({o, dO, delta}, 16));
  const Sizes z = sizes(s, 2);
  FA_TRY(fa::check_alias({{o, z.tensor}, {dO, z.tensor}}, {{delta, z.rows}}));
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_bwd_pre_bf16(o, dO, delta, s.rows(), d, as_stream(stream)));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                      const void* dO, const float* delta, void* dk, void* dv, int64_t B,
                      int64_t H, int64_t N, int64_t d, float scale, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(fa::check_shape(s, true));
  FA_TRY(fa::check_scale(scale));
  if (s.empty()) return FA_OK;
  FA_TRY(fa::check_ptrs({q, k, v, lse, dO, delta, dk, dv}, 16));
  const Sizes z = sizes(s, 2);
  FA_TRY(fa::check_alias({{q, z.tensor}, {k, z.tensor}, {v, z.tensor}, {lse, z.rows},
                          {dO, z.tensor}, {delta, z.rows}},
                         {{dk, z.tensor}, {dv, z.tensor}}));
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_bwd_dkdv_bf16(q, k, v, lse, dO, delta, dk, dv, B * H, N, d, scale,
                                           as_stream(stream)));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                    const void* dO, const float* delta, void* dq, int64_t B, int64_t H,
                    int64_t N, int64_t d, float scale, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(fa::check_shape(s, true));
  FA_TRY(fa::check_scale(scale));
  if (s.empty()) return FA_OK;
  FA_TRY(fa::check_ptrs({q, k, v, lse, dO, delta, dq}, 16));
  const Sizes z = sizes(s, 2);
  FA_TRY(fa::check_alias({{q, z.tensor}, {k, z.tensor}, {v, z.tensor}, {lse, z.rows},
                          {dO, z.tensor}, {delta, z.rows}},
                         {{dq, z.tensor}}));
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_bwd_dq_bf16(q, k, v, lse, dO, delta, dq, B * H, N, d, scale,
                                         as_stream(stream)));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dO, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                 float scale, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, s, scale, true));
  if (s.empty()) return FA_OK;
  float* delta = static_cast<float*>(workspace);
  hipStream_t st = as_stream(stream);
  FA_ON_STREAM_DEVICE(st);
  FA_TRY(from_hip(fa::launch_bwd_pre_bf16(o, dO, delta, s.rows(), d, st)));
  FA_TRY(from_hip(fa::launch_bwd_dkdv_bf16(q, k, v, lse, dO, delta, dk, dv, B * H, N, d, scale, st)));
  return from_hip(fa::launch_bwd_dq_bf16(q, k, v, lse, dO, delta, dq, B * H, N, d, scale, st));
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                         fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(fa::check_shape(s, true));
  FA_TRY(fa::check_scale(scale));
  if (s.empty()) return FA_OK;
  if (s.rows() > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  FA_TRY(fa::check_ptrs({q, k, v, o, dO, dq, dk, dv, lse}, 16));
  const Sizes z = sizes(s, 2);
  FA_TRY(fa::check_alias({{q, z.tensor}, {k, z.tensor}, {v, z.tensor}, {o, z.tensor},
                          {lse, z.rows}, {dO, z.tensor}},
                         {{dq, z.tensor}, {dk, z.tensor}, {dv, z.tensor}}));
  hipStream_t st = as_stream(stream);
  FA_ON_STREAM_DEVICE(st);
  int dev = -1;   // the stream's device, current from here on
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  float* delta = nullptr;
  FA_TRY(scratch_on(dev, &delta));
  // Rows [0, B*H*N) of the scratch are written by the preprocess kernel
  // before the other two read them (in stream order); nothing needs to start
  // at zero.
  FA_TRY(from_hip(fa::launch_bwd_pre_bf16(o, dO, delta, s.rows(), d, st)));
  FA_TRY(from_hip(fa::launch_bwd_dkdv_bf16(q, k, v, lse, dO, delta, dk, dv, B * H, N, d, scale, st)));
  return from_hip(fa::launch_bwd_dq_bf16(q, k, v, lse, dO, delta, dq, B * H, N, d, scale, st));
}

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_fwd(q, k, v, o, lse, s, scale, false));
  if (s.empty()) return FA_OK;
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, scale, as_stream(stream)));
}

int64_t fa_f32_key_block(int64_t N, int64_t d) {
  if (N < 0 || d < 1 || d > 128) return -1;
  return fa::f32_key_block(N, d);
}

size_t fa_bwd_f32_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return fa::bwd_workspace_bytes(Shape{B, H, N, d}, false);
}

fa_status fa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                     const float* lse, const float* dO, float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                     int64_t d, float scale, fa_stream_t stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, s, scale, false));
  if (s.empty()) return FA_OK;
  FA_ON_STREAM_DEVICE(as_stream(stream));
  return from_hip(fa::launch_bwd_f32(q, k, v, o, lse, dO, dq, dk, dv,
                                     static_cast<float*>(workspace), B * H, N, d, scale,
                                     as_stream(stream)));
}

}  // extern "C"
