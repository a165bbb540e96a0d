/*
 * fa2.h - C ABI of the FlashAttention-2 forward library for AMD Instinct MI355X (gfx950).
 *
 * Operation (one call):
 *   For every batch b < B and head h < H, with S = scale * Q[b,h] * K[b,h]^T (N x N):
 *     O[b,h]   = softmax_rows(S masked) * V[b,h]
 *     LSE[b,h,i] = log( sum over visible keys j of exp(S[i,j]) )       (natural log)
 *   Without the causal flag every key is visible to every query.  With it, key j
 *   is visible to query i iff j <= i (queries and keys share one sequence, so
 *   the mask is the square lower triangle).  The N x N score matrix is never
 *   written to memory.
 *
 *   Definition and statistic: "FlashAttention-2 MMA 代码学习" (chuoer47.github.io),
 *   step 0 (O = softmax(Q K^T scale) V) and step 1 (online (m, l) merge);
 *   "第 15 章 FA2 前向：Tiling 与 Online Softmax" (yangyitao.com), §15.1 change 4
 *   (one statistic L = m + log l per row) and the §15.3 kernel skeleton
 *   (signature Q, K, V, O, LSE over [B, H, N, d], softmax_scale, is_causal;
 *   scale before the max; causal mask; ragged N; a row with no visible key
 *   gives O = 0 and LSE = +inf).
 *
 * Layouts (all contiguous, row-major, innermost dimension last):
 *   Q, K, V, O : [B, H, N, d] elements of `dtype` (IEEE binary16 or bfloat16).
 *   LSE        : [B, H, N] float32.
 *
 * Numerics: scores, row statistics and the output accumulator are fp32; the
 * probabilities are rounded (to nearest even) to `dtype` before the second
 * matrix product, as are the outputs.  `scale` may be any finite float,
 * including 0 and negative values.  The exponent base of a row is moved
 * lazily (a probability may exceed 1 by a bounded factor before the row is
 * rescaled), so the fp32 accumulator of O holds at most 2^64 (bf16) or
 * N * 2^16 (fp16) times max|V|: O is finite for finite inputs, given every
 * |V| below 2^64 for bf16 (fp16 values are below 2^16 anyway).
 *
 * Ownership: the caller allocates and owns all five buffers.  The library
 * allocates no device memory and keeps no pointer after the call returns.  Its
 * only mutable global state is the scratch array of fa2_bwd_noalloc (below).
 * Q, K, V are read only; O and LSE are fully overwritten (every element, rows
 * 0..N-1).  O and LSE must not overlap Q, K, V or each other.
 *
 * Execution: the call validates its arguments on the host, then enqueues one
 * kernel on `stream` (a hipStream_t; NULL means the null stream) and returns
 * without synchronising.  It is safe to call from several host threads.
 *
 * Errors: the return value is a status code; nothing is thrown across the ABI.
 * All argument checks run before any HIP call, so a rejected call enqueues
 * nothing and leaves O and LSE untouched.  A launch failure reported by the HIP
 * runtime returns FA2_ERR_HIP.
 */
#ifndef FA2_H_
#define FA2_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA2_DTYPE_FP16 = 0, /* IEEE 754 binary16 */
  FA2_DTYPE_BF16 = 1  /* bfloat16 */
} fa2_dtype_t;

typedef enum {
  FA2_OK = 0,
  FA2_ERR_NULL_POINTER = 1,         /* a buffer pointer is NULL                            */
  FA2_ERR_BAD_SHAPE = 2,            /* B, H or N < 1, or a size limit below is exceeded      */
  FA2_ERR_UNSUPPORTED_HEAD_DIM = 3, /* d is not 32, 64, 96, 128, 256, 512 or 1024            */
  FA2_ERR_UNSUPPORTED_DTYPE = 4,    /* dtype is not FA2_DTYPE_FP16 or FA2_DTYPE_BF16         */
  FA2_ERR_BAD_SCALE = 5,            /* scale is NaN or infinite                              */
  FA2_ERR_MISALIGNED = 6,           /* a [B,H,N,d] tensor not 16-byte aligned, LSE, key_lens
                                       or the workspace not 4-byte aligned                  */
  FA2_ERR_OVERLAP = 7,              /* an output overlaps an input or another output        */
  FA2_ERR_HIP = 8,                  /* the HIP runtime reported an error at launch           */
  FA2_ERR_TOO_LARGE = 9             /* fa2_bwd_noalloc: B * H * N above its scratch (2^21)   */
} fa2_status_t;

/*
 * fa2_fwd - attention forward with log-sum-exp, as described above.
 *
 *   Q, K, V   device pointers to [B, H, N, d] `dtype` tensors (read only).
 *   O         device pointer to a [B, H, N, d] `dtype` tensor (written).
 *   LSE       device pointer to a [B, H, N] float32 tensor (written).
 *   B, H, N   batch, heads, sequence length; each >= 1.  Limits, with R the
 *             query rows per workgroup (256 for d = 64 and 128, 128 for
 *             d = 32, 96, 256 and 512, 64 for d = 1024; d = 128 takes a
 *             128-row form on grids of at most one 256-row workgroup per
 *             compute unit, which fa2_launch_info reports, and the limit
 *             below uses 256):
 *             (N + 256) * d * 2 < 2^31 (one head's slice, with the rows past
 *             N that the last query tile and the last key tiles touch, is
 *             addressed with signed 32-bit byte offsets) and
 *             ceil(N / R) * H * B < 2^31 (grid size).
 *   d         head dimension: 32, 64, 96, 128, 256, 512 or 1024.
 *   scale     softmax scale applied to Q K^T before the row max; any finite value.
 *   is_causal 0: all keys visible; nonzero: key j visible to query i iff j <= i.
 *   dtype     element type of Q, K, V and O (fa2_dtype_t).
 *   stream    hipStream_t to enqueue on; NULL is the null stream.
 */
fa2_status_t fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int is_causal,
                     int dtype, void* stream);

/*
 * fa2_fwd_masked - fa2_fwd under a sliding window and per-sequence key
 * lengths (right padding).  The pages name sliding-window and padding masks
 * as the masks under which a row can see only hidden keys in its first key
 * tiles, which is what the kernel's -inf guards are for ("第 15 章 FA2 前向：
 * Tiling 与 Online Softmax", the note after the §15.3 kernel skeleton); their
 * form here is this library's reading:
 *
 *   key j is visible to query i of batch b iff
 *       j <  key_lens[b]            (when key_lens is not NULL)
 *       j >= i - window_left        (when window_left >= 0)
 *       j <= i + window_right       (when window_right >= 0)
 *
 * and the softmax runs over the visible keys only.  A row with no visible
 * key gets O = 0 and LSE = +inf.  window_left < 0 with window_right = 0 is
 * the causal mask of fa2_fwd; a bound >= N hides nothing.
 *
 *   window_left, window_right  window bounds in keys; negative: no bound.
 *   key_lens  NULL (no padding) or a device pointer to B int32 lengths, read
 *             by the kernel (4-byte aligned; must not overlap O or LSE);
 *             values outside [0, N] are clamped to it.  K and V rows at or
 *             past the length are never read (they may hold anything, NaN
 *             included); keys hidden by the window are read and must be
 *             finite, as every key of fa2_fwd must.
 *   All other arguments, checks, limits and status codes are those of
 *   fa2_fwd.  A call with no window runs fa2_fwd's unmasked kernel and a
 *   call with window (<0, 0) its causal kernel, with or without key_lens
 *   (without them the results are bit-identical to fa2_fwd's); every other
 *   call runs the general-mask kernel.
 */
fa2_status_t fa2_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                            int64_t window_left, int64_t window_right, const int32_t* key_lens,
                            int dtype, void* stream);

/*
 * fa2_bwd - gradients of the attention of fa2_fwd (no window, no key
 * lengths): given dO = dL/dO for some loss L, writes dQ, dK and dV.  With S
 * and P = exp(S - LSE) as above (the forward's probabilities, recomputed
 * from Q, K and the forward's LSE):
 *
 *   dV    = P^T dO
 *   dP    = dO V^T,   Delta_i = sum_d dO[i,d] O[i,d],   dS = P * (dP - Delta)
 *   dQ    = scale * dS K,   dK = scale * dS^T Q
 *
 *   The backward the pages outline: "第 15 章 FA2 前向：Tiling 与 Online
 *   Softmax" (yangyitao.com), the chapter's closing paragraph (S and P
 *   recomputed from the stored statistic, keys in the outer loop); the
 *   arithmetic is the chain rule through the softmax of the definition above.
 *
 *   Q, K, V, O, dO  device pointers to [B, H, N, d] `dtype` tensors (read
 *             only); O and LSE are the outputs of fa2_fwd for the same Q, K,
 *             V, scale and is_causal (any O and LSE are accepted: they enter
 *             the formulas above as given).
 *   LSE       device pointer to the [B, H, N] float32 LSE of fa2_fwd.
 *   dQ, dK, dV  device pointers to [B, H, N, d] `dtype` tensors (written,
 *             every element).
 *   workspace device pointer to 2 * B * H * N float32 values of scratch,
 *             owned by the caller; its contents on entry do not matter.  When
 *             the call's work has run it holds -Delta of every row ([B, H, N])
 *             followed by -LSE * log2(e) of every row ([B, H, N]).
 *   B, H, N, scale, is_causal, dtype, stream: as for fa2_fwd, with d = 32,
 *             64, 96, 128 or 256 only, and ceil(N / 128) * H * B < 2^31.
 *
 * Numerics: S, dP, Delta and the accumulators are fp32; P and dS are rounded
 * to `dtype` (to nearest even) before the products that take them, and the
 * gradients once at the end.  P <= 1 needs no guard; with fp16 the rounded
 * dS = P (dP - Delta) must stay below 65504 in magnitude (dP is a dot
 * product of dO and V rows), else dQ and dK of that row and key are not
 * finite.  The call enqueues two kernels on `stream`
 * (first dQ and the row statistics, then dK and dV), allocates nothing and does not
 * synchronise.  Errors: as for fa2_fwd; FA2_ERR_OVERLAP when dQ, dK, dV or
 * the workspace overlaps an input or one another; FA2_ERR_UNSUPPORTED_HEAD_DIM
 * for d other than 32, 64, 96, 128 and 256.
 */
fa2_status_t fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int is_causal,
                     int dtype, void* stream);

/*
 * fa2_bwd_masked - fa2_bwd for the attention of fa2_fwd_masked: the same
 * window and key-length arguments, the same visibility of keys, and O and LSE
 * from fa2_fwd_masked.  A row with no visible key (LSE = +inf) gets dQ = 0
 * and adds nothing to dK and dV; keys at or past a sequence's length get
 * dK = dV = 0 and their K and V rows are never read.  The gradients are
 * those of the masked definition (the same chain rule with P the softmax
 * over each row's visible keys; reading of the pages as for
 * fa2_fwd_masked).  All other arguments, checks, limits and status codes
 * are those of fa2_bwd (key_lens: as for fa2_fwd_masked, 4-byte aligned,
 * not overlapping an output).  No window and no key lengths run fa2_bwd's
 * unmasked kernels, window (<0, 0) without key lengths its causal ones.
 */
fa2_status_t fa2_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                            const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                            int64_t window_left, int64_t window_right, const int32_t* key_lens,
                            int dtype, void* stream);

/*
 * fa2_bwd_noalloc - fa2_bwd without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a scratch array inside
 * the library (one per GPU, 2^22 floats, held until the process ends); the
 * call allocates nothing.  B * H * N above 2^21 returns FA2_ERR_TOO_LARGE (before
 * anything is enqueued).  Every call on one GPU shares that GPU's array: calls
 * whose work overlaps in time on one GPU (on different streams, or from
 * different host threads without ordering) race on it and give undefined
 * results; calls ordered on one stream do not.  The workspace is fully rewritten by
 * each call before it is read, so nothing needs clearing.  Results are
 * bit-identical to fa2_bwd's (same kernels).  All other arguments, checks and
 * status codes are those of fa2_bwd.
 */
fa2_status_t fa2_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int is_causal,
                             int dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa2_status_string(int status);

/*
 * fa2_launch_info - the launch fa2_fwd would make for these arguments, without
 * launching.  Writes the number of workgroups, threads per workgroup, query
 * rows per workgroup, keys per tile and LDS bytes per workgroup.  Returns the
 * status fa2_fwd would return from its argument checks (pointers are not
 * examined).  Any output pointer may be NULL.  For d = 32, 64 and 128 the
 * form of the launch (threads, rows, LDS bytes) depends on how many
 * workgroups the grid gives each compute unit of the current device (queried
 * once per device; 256 compute units are assumed when no device can be
 * queried), and at d = 128 also on the mask.
 */
fa2_status_t fa2_launch_info(int64_t B, int64_t H, int64_t N, int64_t d, int is_causal, int dtype,
                             int64_t* workgroups, int* threads, int* rows_per_wg,
                             int* keys_per_tile, int* lds_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H_ */
