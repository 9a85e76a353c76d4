/* evo_attn.h — C ABI of the MI355X (gfx950) Evoformer biased attention library.
 *
 * The operation is the one the DeepSpeed4Science guide describes for
 * DS4Sci_EvoformerAttention (page "DeepSpeed4Science 技术指南"):
 *   §3.5  reference attention: QK^T times the scale factor, plus the bias,
 *         softmax over keys, times V;
 *   §3.6  the tensor layouts of MSA row, MSA column and triangle attention:
 *         Q, K, V [B, N, L, H, D]; bias 1 (a residue mask) [B, N, 1, 1, L];
 *         bias 2 (pair bias / edges) [B, 1, H, L, L];
 *   §3.7  at most two biases, a missing one treated as absent; the forward
 *         keeps O and an fp32 log-sum-exp per query row; the backward derives
 *         delta from them and returns the gradients of Q, K, V and of both
 *         biases, the bias gradients accumulated in fp32 and cast back to the
 *         input dtype; the backward supports head dims up to 64.
 *
 *   S[b,n,h,i,j] = scale * sum_d Q[b,n,i,h,d] K[b,n,j,h,d] + mask[b,n,j] + pair[b,h,i,j]
 *   O[b,n,i,h,:] = sum_j softmax_j(S)[b,n,h,i,j] V[b,n,j,h,:]
 *   lse[b,n,h,i] = log sum_j exp S[b,n,h,i,j]          (natural log, fp32)
 *   scale = 1/sqrt(D).
 *
 * Conventions common to every entry point
 *   - shape = {B, N, L, H, D}; B, N, L, H >= 1; D in {8, 16, 32, 64}.
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device, to
 *     a dense row-major buffer, 16-byte aligned (the _strided entry points
 *     take other layouts for the [B,N,L,H,D] tensors).  16-bit tensors hold IEEE
 *     half (EVO_F16) or bfloat16 (EVO_BF16) values; lse is float32.
 *   - All buffers are owned by the caller.  The library allocates no device
 *     memory and keeps no state between calls; calls are re-entrant.  The one
 *     exception is evo_attn_bwd_noalloc, whose workspace is a static device
 *     array of EVO_NOALLOC_SCRATCH_BYTES that every GPU holds while the library
 *     is loaded.
 *   - Outputs are overwritten, never accumulated.  No output may alias an
 *     input or another output.
 *   - A bias pointer may be NULL: that bias is absent (treated as zero).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream) and the call returns without waiting for it.
 *   - Argument errors are detected on the host before anything is enqueued:
 *     the call returns a non-zero status and leaves every output untouched.
 *     A launch failure returns EVO_ERR_LAUNCH.  The library never aborts and
 *     never prints.
 */
#ifndef EVO_ATTN_H
#define EVO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { EVO_F16 = 0, EVO_BF16 = 1 } evo_dtype_t;

typedef enum {
  EVO_OK = 0,
  EVO_ERR_NULL_POINTER = 1,      /* a required pointer is NULL, or a bias gradient was requested without its bias */
  EVO_ERR_BAD_SHAPE = 2,         /* a dimension < 1, or sizes that overflow 32-bit indexing */
  EVO_ERR_BAD_DTYPE = 3,         /* dtype is neither EVO_F16 nor EVO_BF16 */
  EVO_ERR_HEAD_DIM = 4,          /* D not in {8, 16, 32, 64} */
  EVO_ERR_ALIGNMENT = 5,         /* a pointer is not 16-byte aligned */
  EVO_ERR_NOT_DEVICE_MEMORY = 6, /* a pointer is not device memory of the current device */
  EVO_ERR_WORKSPACE = 7,         /* workspace NULL or smaller than evo_attn_bwd_workspace_bytes_within(..., 0) */
  EVO_ERR_DEVICE = 8,            /* the current device is not gfx950 */
  EVO_ERR_LAUNCH = 9,            /* a kernel launch failed */
  EVO_ERR_ALIAS = 10,            /* an output overlaps an input or another output */
  EVO_ERR_BAD_STRIDES = 11,      /* strides not multiples of 8, rows that overlap, or a slice past 2 GiB */
  EVO_ERR_SCRATCH_LIMIT = 12     /* evo_attn_bwd_noalloc: the problem needs more than EVO_NOALLOC_SCRATCH_BYTES */
} evo_status_t;

/* Forward (guide §3.5 and §3.7: fused attention that keeps O and the fp32 lse).
 *   q, k, v     [B,N,L,H,D] dtype          inputs
 *   mask_bias   [B,N,1,1,L] dtype or NULL  additive bias on keys, shared by all heads and queries
 *   pair_bias   [B,1,H,L,L] dtype or NULL  additive bias, shared by every n
 *   out         [B,N,L,H,D] dtype          output
 *   lse         [B,N,H,L]   float32        natural-log log-sum-exp of each row of S, or NULL
 * A query row whose scores are all -inf gets out = 0 and lse = -inf.  A key whose mask
 * bias is -inf (fp16's rounding of -1e9, or an explicit -inf) has P = 0 in every row: it
 * adds nothing to out, lse, dq or dpair, and gets dk = dv = dmask = 0.  The 32-key blocks
 * past the last key of a key tile (256 keys, 128 at D = 64) that is not -inf are not
 * computed, and on the key side of the backward neither is a group of 16 keys that are all
 * -inf, so a padded batch masked with -inf costs less than its full length (the
 * block-sparse principle of the page "DeepSpeed Sparse Attention 深度解析", section
 * 核心思想: only the blocks a mask leaves are computed; applied here to padding).  A
 * finite mask, however large, is computed.  A pair_bias entry of -inf makes that score
 * -inf (P = 0 there), as the mask does for a whole key.  With lse NULL the
 * call is a forward for inference (the guide's §3.2 notes the forward kernels pay off
 * at inference for every attention type): out is the same, bit for bit, and nothing is
 * kept for a backward. */
evo_status_t evo_attn_fwd(const void* q, const void* k, const void* v, const void* mask_bias,
                          const void* pair_bias, void* out, float* lse, const int64_t shape[5],
                          int dtype, void* stream);

/* Bytes of device workspace for evo_attn_bwd on this problem (0 on bad
 * arguments): fp32 delta and bias-gradient accumulators, the dpair partials of
 * the slice groups and, for rows longer than one key tile (L > 256, or > 128
 * at D = 64) with a pair bias, the fp32 dQ partials of each key tile (without
 * a pair bias the query side keeps dQ in registers over all key tiles and
 * needs no partials).  The backward fits its plan to the workspace it is
 * given: with less room it takes the slices of long rows in chunks (more
 * launches, smaller partials).  This size is that
 * of the plan with at most 384 MiB of partials; evo_attn_bwd_workspace_bytes_within
 * gives the size for another bound on the partials (0: the least workspace
 * the backward accepts).  The workspace size is an input of the plan: the bias
 * gradients' summation order, hence their last bits, can depend on it, and a
 * call is bitwise reproducible for the same arguments. */
size_t evo_attn_bwd_workspace_bytes(const int64_t shape[5], int dtype, int has_mask, int has_pair);
size_t evo_attn_bwd_workspace_bytes_within(const int64_t shape[5], int dtype, int has_mask, int has_pair,
                                           size_t partial_budget);

/* Byte offsets into the workspace, valid after evo_attn_bwd returns and its
 * work completes, of the fp32 accumulators the bias gradients are cast from:
 *   delta      [B,N,H,L]   rowsum(dO * O)
 *   dmask_f32  [B,N,L]     sum over h and i of dS          (only if has_mask)
 *   dpair_f32  [B,H,L,L]   sum over n of dS                (only if has_pair)
 * An offset is set to (size_t)-1 when that accumulator is absent.
 * Returns EVO_OK or an argument error. */
evo_status_t evo_attn_bwd_workspace_offsets(const int64_t shape[5], int dtype, int has_mask,
                                            int has_pair, size_t* off_delta, size_t* off_dmask_f32,
                                            size_t* off_dpair_f32);

/* Backward (guide §3.7: recompute from lse, derive delta, then the gradients).
 *   q, k, v, mask_bias, pair_bias  as passed to evo_attn_fwd
 *   out, lse                       exactly as evo_attn_fwd wrote them
 *   dout        [B,N,L,H,D] dtype  gradient of the loss w.r.t. out
 *   dq, dk, dv  [B,N,L,H,D] dtype  outputs
 *   dmask_bias  [B,N,1,1,L] dtype  output: sum over h and i of dS; may be NULL (not computed)
 *   dpair_bias  [B,1,H,L,L] dtype  output: sum over n of dS;       may be NULL (not computed)
 *   workspace, workspace_bytes     device scratch of at least evo_attn_bwd_workspace_bytes_within(..., 0)
 *                                  (evo_attn_bwd_workspace_bytes() for the default plan), contents
 *                                  undefined on entry; see evo_attn_bwd_workspace_offsets
 * The bias gradients are accumulated in fp32 in a fixed order (the result
 * is bitwise reproducible) and rounded to dtype to nearest even.
 * Passing dmask_bias without mask_bias, or dpair_bias without pair_bias, is
 * EVO_ERR_NULL_POINTER. */
evo_status_t evo_attn_bwd(const void* q, const void* k, const void* v, const void* mask_bias,
                          const void* pair_bias, const void* out, const float* lse, const void* dout,
                          void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias,
                          void* workspace, size_t workspace_bytes, const int64_t shape[5], int dtype,
                          void* stream);

/* The same operations on [B,N,L,H,D] tensors laid out with element strides
 * strides = {sB, sN, sL} for dims B, N, L, shared by every such tensor of the
 * call (q, k, v, out; and dout, dq, dk, dv for the backward); within one
 * (b, n, l) row the H heads of D elements are dense.  Guide §3.6 names triangle
 * attention around the ending node beside the starting-node form it shows:
 * with sN and sL exchanged it runs on a view of the pair representation
 * transposed over its two residue axes, without a copy.  Requirements (else
 * EVO_ERR_BAD_STRIDES, before any device call): every stride a positive
 * multiple of 8 elements; no two rows overlap (over the dims of extent > 1 in
 * increasing stride order, each stride at least the span of the ones below
 * it, the first at least H * D); (L - 1) * sL + H * D elements of one slice
 * under 2 GiB.  strides == NULL is the dense layout {N*L*H*D, L*H*D, H*D}:
 * evo_attn_fwd and evo_attn_bwd are these calls with NULL strides.  mask_bias,
 * pair_bias, lse, their gradients and the workspace keep their dense layouts.
 * Output values do not depend on the strides (bit for bit). */
evo_status_t evo_attn_fwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, void* out, float* lse, const int64_t shape[5],
                                  const int64_t strides[3], int dtype, void* stream);
evo_status_t evo_attn_bwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias,
                                  void* workspace, size_t workspace_bytes, const int64_t shape[5],
                                  const int64_t strides[3], int dtype, void* stream);

/* The backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and results are those of evo_attn_bwd_strided (strides NULL: the
 * dense layout) without the workspace: the call allocates nothing and uses
 * instead a static device array of EVO_NOALLOC_SCRATCH_BYTES bytes (64 MiB)
 * that every GPU the library runs on holds until the process ends, with the
 * plan fitted to it as to a workspace of that size.  A problem whose
 * evo_attn_bwd_workspace_bytes_within(..., 0) exceeds that limit returns
 * EVO_ERR_SCRATCH_LIMIT before anything is enqueued.  All calls on one GPU
 * share its array, which keeps the last call's contents: calls that overlap
 * on one GPU (on different streams, or from several threads) race and must be
 * serialised by the caller.  The fp32 accumulators that
 * evo_attn_bwd_workspace_offsets describes are not reachable through this call. */
#define EVO_NOALLOC_SCRATCH_BYTES (64u << 20)
evo_status_t evo_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias,
                                  const int64_t shape[5], const int64_t strides[3], int dtype, void* stream);

/* Static text for a status code (never NULL). */
const char* evo_status_string(int status);

/* ---- Optional instrumentation (measurement only; does not change results).
 * When enabled, the library records a pair of hipEvents on the caller's stream
 * around each of its kernel launches; evo_attn_profile_read waits for the
 * recorded launches and returns, per kernel kind, the summed elapsed time and
 * the launch count since the previous read, then forgets them.
 * Kinds: 0 fwd, 1 bwd_pre (delta), 2 bwd_kv (dK, dV, dmask partials),
 *        3 bwd_q (dQ, dpair partials), 4 bwd_fin (bias-gradient reductions).
 * At most 65536 launches are kept between reads; later ones are not recorded. */
#define EVO_PROFILE_KINDS 5
int evo_attn_profile_enable(int on); /* returns the previous setting */
evo_status_t evo_attn_profile_read(double total_ms[EVO_PROFILE_KINDS], int64_t launches[EVO_PROFILE_KINDS]);
const char* evo_attn_profile_kernel_name(int kind); /* static text, never NULL */

#ifdef __cplusplus
}
#endif

#endif /* EVO_ATTN_H */
