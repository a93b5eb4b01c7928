/*
 * fa.h -- libfa: exact FlashAttention forward pass for AMD Instinct MI355X
 * (gfx950), C ABI.
 *
 * The operation.  For each batch b, head h and query row i,
 *     O_i   = sum_j softmax_j(scale * q_i . k_j) * v_j
 *     LSE_i = log sum_j exp(scale * q_i . k_j)          (natural log)
 * over the visible keys j: all j in [0, N), or j <= i when `causal` is set.
 * The result is computed tile by tile with the online-softmax recurrence
 * (a running row maximum and a running sum of exponentials, with earlier
 * partial results rescaled whenever the maximum grows, and one division by
 * the sum at the end), so the N x N score matrix never reaches memory.
 * Sources:
 *   - "FlashAttention dissected" (leren.llmnet.nl): sections "The
 *     mathematical breakthrough: Tiling and Online Softmax" (softmax of a row,
 *     rescaling by exp(m_old - m_new)), "FlashAttention-1 versus
 *     FlashAttention-2" (query blocks outside, independent thread blocks),
 *     "Memory complexity" (the row statistics m and l are what the backward
 *     pass keeps; LSE = m + ln l carries both) and "Algorithmic core in
 *     pseudocode" (the recurrence and the final division by l);
 *   - "How Did I Write My First FlashAttention Kernel in CUDA?": the tiled
 *     pseudo-algorithm (Q/O blocks of B_r x d, K/V blocks of B_c x d, m
 *     initialised to -inf and l to 0);
 *   - "CUDA Flash Attention: Online Softmax with Shared Memory Tiling"
 *     (GitHub README), "Design decisions": scale passed in by the caller,
 *     masking of out-of-range keys, the guard against -inf - (-inf) for rows
 *     whose scores are all masked, 64-bit indexing, restrict-qualified
 *     (non-aliasing) pointers and error surfacing after the launch.
 * The causal mask (key j > query i is masked) is not defined by the pages;
 * it is the convention of the causal workloads this library is measured on.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  Accumulation is always fp32. */
typedef enum {
  FA_F32 = 0,  /* IEEE binary32 in, fp32 MFMA, fp32 out            */
  FA_BF16 = 1, /* bfloat16 in, bf16 MFMA into fp32, bfloat16 out   */
  FA_F16 = 2   /* binary16 in, fp16 MFMA into fp32, binary16 out    */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,     /* q, k, v or o is NULL                                  */
  FA_ERR_SHAPE = 2,    /* B, H or N negative, or the problem is too large       */
  FA_ERR_HEAD_DIM = 3, /* d is not one of the supported head sizes (64, 128)    */
  FA_ERR_DTYPE = 4,    /* dtype is not an fa_dtype value                        */
  FA_ERR_SCALE = 5,    /* scale is not finite or not > 0                        */
  FA_ERR_ALIGN = 6,    /* q, k, v or o not 16-byte aligned, lse not 4-byte      */
  FA_ERR_ALIAS = 7,    /* o or lse overlaps another buffer                      */
  FA_ERR_LAUNCH = 8    /* the HIP runtime refused the kernel launch             */
} fa_status;

/*
 * fa_fwd -- O = softmax(Q K^T * scale) V and the per-row logsumexp.
 *
 * q, k, v  device pointers to contiguous row-major [B, H, N, d] arrays of
 *          `dtype` (element (b, h, i, c) at ((b*H + h)*N + i)*d + c).  They
 *          are only read and may alias one another.
 * o        device pointer to a contiguous [B, H, N, d] array of `dtype`,
 *          written in full (rows are rounded to nearest-even from fp32).
 * lse      device pointer to a contiguous fp32 [B, H, N] array, written in
 *          full, or NULL to skip it.  LSE_i = scale * m_i + ln(l_i) in natural
 *          log; a row with no visible key would get O_i = 0, LSE_i = -inf.
 * B, H, N  batch, heads, sequence length (queries = keys = N).  Any of them
 *          zero is a valid empty problem and returns FA_OK with no launch.
 *          Limits (else FA_ERR_SHAPE): B*H <= 2^31-1, one head's N x d
 *          array (plus 256 rows) below 2^31 bytes, and the launch grid
 *          (B*H*ceil(N/128) workgroups) below 2^31.
 * d        head dimension: 64 or 128.
 * scale    multiplier of the dot products (usually 1/sqrt(d)); finite, > 0.
 * causal   nonzero: key j is masked for query i when j > i.
 * stream   hipStream_t to launch on (NULL = the default stream).
 *
 * Ownership: the caller owns every buffer.  The library allocates no device
 * or host memory, keeps no pointer after returning and holds no mutable
 * global state, so concurrent calls from several host threads are safe.
 *
 * Ordering and errors: arguments are validated on the host before anything
 * touches the GPU; a bad argument returns its status and launches nothing.
 * One kernel is then enqueued on `stream` and the call returns without
 * waiting: results are valid once the caller synchronises that stream.
 * FA_ERR_LAUNCH reports a launch the runtime refused; faults during
 * execution surface at the caller's next synchronisation.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                 fa_dtype dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(fa_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
