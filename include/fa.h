/*
 * fa.h - C ABI of an exact, IO-aware scaled-dot-product attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch b and head h, with S = scale * Q K^T:
 *     O   = softmax(S) V                          (forward)
 *     LSE = ln sum_j exp(S_ij)   (one fp32 per query row, natural log)
 *     dQ, dK, dV = gradients of sum(O * dO)      (backward)
 * The formula is the scaled dot-product attention of the star-observatory
 * FlashAttention fable page (ckw19810413.github.io, section 概念揭曉).  The
 * forward tiles Q, K and V and keeps the running max, running sum and output
 * on chip, rescaling by exp(m_old - m_new) (same page, section "兩大核心魔法";
 * 账房先生的奔命 (carrie-l.github.io), section 六), so no N x N matrix is
 * ever written to device memory.  The backward recomputes P from Q, K and
 * the saved LSE instead of storing it (账房先生的奔命, section 七).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer.  Q, K, V, O, dO, dQ, dK, dV are
 *     contiguous [B][H][N][d] (d fastest); LSE is [B][H][N] float32.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates device memory and keeps no state between calls; calls
 *     are reentrant.
 *   - Outputs are fully overwritten (never accumulated into) and must not
 *     overlap any input or each other (FA_ERR_ALIAS).
 *   - `stream` is a hipStream_t (NULL = the null stream of the current
 *     device).  Work is enqueued asynchronously; nothing synchronises with
 *     the host.  The kernels run on the stream's device, which the call
 *     makes current while it launches and then restores the caller's; the
 *     tensors must be on that device.
 *   - Arguments are checked before anything is enqueued.  A return other than
 *     FA_OK or FA_ERR_HIP means nothing was enqueued.  A launch failure is
 *     FA_ERR_HIP; launches of the same call made before it stay enqueued and
 *     the outputs are then unspecified.  Faults during execution surface at
 *     the caller's next synchronisation.
 *   - Sizes set no grid limit of their own: a kernel whose grid would exceed
 *     2^31 work-items is launched in several chunks of whole heads (or of
 *     whole blocks of rows), since a single dispatch of 2^32 work-items or
 *     more is cut short by the runtime without an error.  Only a grid of one
 *     head that alone exceeds 2^31 work-items is refused, FA_ERR_SHAPE: the
 *     fp32 calls on key blocks of 8 with N > 2^28, and fa_fwd_split with
 *     n_split * ceil(N/256) > 2^22.
 *   - B, H or N equal to 0 is an empty problem: FA_OK, nothing enqueued, and
 *     pointers may be NULL.  Negative sizes are FA_ERR_SHAPE.
 *   - `scale` must be finite and > 0 (FA_ERR_SCALE); 1/sqrt(d) rounded to
 *     float is the usual value.
 *   - No C++ exception crosses this boundary and the library prints nothing.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  FA_ERR_SHAPE = 2,       /* a size is negative, or offsets overflow          */
  FA_ERR_UNSUPPORTED = 3, /* head dim not supported by this entry point        */
  FA_ERR_ALIGN = 4,       /* a pointer is not aligned as required              */
  FA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  FA_ERR_SCALE = 6,       /* scale not finite or not > 0                       */
  FA_ERR_ALIAS = 7,       /* an output overlaps an input or another output     */
  FA_ERR_HIP = 8,         /* the HIP runtime rejected a launch                 */
  FA_ERR_SCRATCH = 9      /* problem larger than a fixed scratch array         */
} fa_status;

/* A hipStream_t, passed as an opaque pointer so this header needs no HIP. */
typedef void* fa_stream_t;

/* Human-readable text for a status; never NULL, static storage. */
const char* fa_status_str(fa_status s);

/* ------------------------------------------------------------------------ */
/* bf16 path: Q, K, V, O, dO, dQ, dK, dV hold bfloat16 (uint16 storage).    */
/* Head dim d must be 64 or 128, and one head of one tensor at most 2 GiB:  */
/* (N + 128) * d * 2 < 2^31 bytes, else FA_ERR_SHAPE.  Tensor pointers, LSE  */
/* and the workspace 16-byte aligned.  Accumulation is fp32 throughout; P    */
/* and dS are rounded to bf16 (round to nearest even) before their           */
/* contractions.                                                              */
/* ------------------------------------------------------------------------ */

/* Forward.  Inputs q, k, v; outputs o (bf16) and lse (fp32, natural log).
 * Tiling and online softmax: 账房先生的奔命, section 六; rescale identity:
 * star-observatory fable page, section "兩大核心魔法"; only O and the row
 * statistic return to memory: 算珠楼的掌簿人 (hespethorn.github.io), 技术解读. */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 fa_stream_t stream);

/* Split-KV forward (more workgroups when B*H is small; also the per-device
 * step of a key-sharded forward).  The keys are cut into n_split contiguous
 * ranges of whole key tiles (128 keys at d = 128, 64 at d = 64): range p
 * holds tiles [p*T/n_split, (p+1)*T/n_split) with T = ceil(N/tile) and
 * integer division, so every range holds at least one tile.  For each range
 * and query row i it writes
 *   lse_part[p][b][h][i]    = ln sum_{j in range p} exp(scale * q_i . k_j)
 *   o_part[p][b][h][i][:]   = sum_{j in range p} exp(scale * q_i . k_j - lse_part) v_j
 * i.e. the forward restricted to the range (fp32 output, normalised by the
 * range's own sum).  o_part is float32 [n_split][B][H][N][d] and lse_part
 * float32 [n_split][B][H][N], both 16-byte aligned.  1 <= n_split <=
 * fa_fwd_split_max(B,H,N,d), else FA_ERR_SHAPE.  Tiling per range as in
 * fa_fwd; the ranges are recombined by fa_merge (star-observatory fable
 * page, section "兩大核心魔法"). */
int64_t fa_fwd_split_max(int64_t B, int64_t H, int64_t N, int64_t d); /* -1: invalid shape */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, float* o_part,
                       float* lse_part, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       int64_t n_split, fa_stream_t stream);

/* Merge of n_split partial results (any source: fa_fwd_split, other
 * devices, ...).  For each row, with m = max_p lse_part[p]:
 *   lse = m + ln sum_p exp(lse_part[p] - m)
 *   o   = sum_p exp(lse_part[p] - lse) * o_part[p]          (bf16 output, RNE)
 * the rescale identity of the star-observatory fable page (section
 * "兩大核心魔法"); the order of the parts does not matter (算珠楼的掌簿人,
 * section 四).  A part with lse_part = -inf contributes nothing (its o_part
 * values are read but not used, so they may be NaN); a row whose parts are
 * all -inf gets o = 0, lse = -inf.
 * o_part float32 [n_split][B][H][N][d], lse_part float32 [n_split][B][H][N]
 * (inputs); o bf16 [B][H][N][d], lse float32 [B][H][N] (outputs).  d must be
 * 64 or 128; 1 <= n_split <= 2^24 (else FA_ERR_SHAPE); 16-byte alignment;
 * outputs may not overlap the inputs (FA_ERR_ALIAS). */
fa_status fa_merge(const float* o_part, const float* lse_part, int64_t n_split, void* o,
                   float* lse, int64_t B, int64_t H, int64_t N, int64_t d, fa_stream_t stream);

/* Bytes of workspace fa_bwd needs: one fp32 per query row (D = rowsum(dO*O)),
 * rounded up to 256.  0 for an empty problem.  (size_t)-1 for invalid sizes. */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/* Backward with recomputation (账房先生的奔命, section 七: P is recomputed from
 * Q, K and the saved LSE, never stored).  Inputs q, k, v, the forward's o and
 * lse, and dO; outputs dq, dk, dv (bf16).  Runs fa_bwd_preprocess,
 * fa_bwd_dkdv and fa_bwd_dq in that order on `stream`; deterministic (no
 * atomics).  `workspace` must hold fa_bwd_workspace_bytes(B,H,N,d) bytes.   */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 fa_stream_t stream);

/* fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same computation, arguments and errors as fa_bwd, without the workspace
 * arguments.  Its workspace (D, one fp32 per query row) is a fixed array the
 * library holds on every GPU it runs on, FA_BWD_NOALLOC_MAX_ROWS rows
 * (16 MiB); B*H*N above that is FA_ERR_SCRATCH.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a device
 * looks up that device's array once.  Every call on one GPU uses the same
 * array: calls that overlap in time on one GPU (different streams, or other
 * threads) race and give wrong gradients; calls ordered on one stream do not.
 * Results are bit-identical to fa_bwd. */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                         fa_stream_t stream);

/* The three stages of fa_bwd, exposed so that each launch can be timed and
 * tested on its own.  `delta` is [B][H][N] fp32 (16-byte aligned).
 * fa_bwd_preprocess: delta_i = sum_c dO_ic * O_ic (the O the forward stored). */
fa_status fa_bwd_preprocess(const void* o, const void* dO, float* delta,
                            int64_t B, int64_t H, int64_t N, int64_t d,
                            fa_stream_t stream);
/* fa_bwd_dkdv: per key tile, recompute P^T from K, Q and lse, then
 * dV = P^T dO and dK = scale * dS^T Q with dS = P * (dO V^T - delta).        */
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                      const void* dO, const float* delta, void* dk, void* dv,
                      int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                      fa_stream_t stream);
/* fa_bwd_dq: per query tile, recompute P and dS and form dQ = scale * dS K.  */
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                    const void* dO, const float* delta, void* dq,
                    int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                    fa_stream_t stream);

/* ------------------------------------------------------------------------ */
/* fp32 path: every tensor is float32, 1 <= d <= 128, pointers 4-byte        */
/* aligned; no rounding anywhere (P and dS stay fp32).  Same method and      */
/* citations as the bf16 calls.  The key block (keys per rescale step) is    */
/* chosen by shape, see fa_f32_key_block: up to N = 256, and for head dims   */
/* other than 64 and 128, FMA kernels step through key blocks of 8 with the  */
/* exact running max (the 64 rows in 8 stacks of 8 of 算珠楼的掌簿人, fable   */
/* section 二, updated by the rule of 账房先生的奔命, section 六); longer      */
/* sequences at d = 64 or 128 run on the fp32 matrix cores with key and      */
/* query tiles of 32 (when one head of one tensor fits 2 GiB).               */
/* ------------------------------------------------------------------------ */

/* Keys per rescale step that fa_fwd_f32 and fa_bwd_f32 use for sequence    */
/* length N and head dim d: 8 or 32.  -1 if N < 0 or d is outside 1..128.   */
/* Pure function of its arguments; launches nothing.                        */
int64_t fa_f32_key_block(int64_t N, int64_t d);

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     fa_stream_t stream);

/* Same sizing rule as fa_bwd_workspace_bytes. */
size_t fa_bwd_f32_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

fa_status fa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                     const float* lse, const float* dO, float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     fa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
