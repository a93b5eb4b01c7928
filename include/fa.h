/*
 * fa.h -- libfa: exact FlashAttention forward and backward passes for AMD
 * Instinct MI355X (gfx950), C ABI.
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
  FA_ERR_NULL = 1,     /* a required pointer (q, k, v, o, partials) is NULL     */
  FA_ERR_SHAPE = 2,    /* a size negative, H not a multiple of H_kv, too large  */
  FA_ERR_HEAD_DIM = 3, /* d is not one of the supported head sizes (64, 128)    */
  FA_ERR_DTYPE = 4,    /* dtype not an fa_dtype value                           */
  FA_ERR_SCALE = 5,    /* scale is not finite or not > 0                        */
  FA_ERR_ALIGN = 6,    /* a tensor not 16-byte aligned, lse not 4-byte          */
  FA_ERR_ALIAS = 7,    /* an output or the workspace overlaps another buffer    */
  FA_ERR_LAUNCH = 8,   /* the HIP runtime refused the kernel launch             */
  FA_ERR_WORKSPACE = 9, /* num_splits < 1, or workspace null, small or misaligned */
  FA_ERR_SCRATCH = 10   /* fa_fwd_ex_noalloc: partials exceed its static scratch */
} fa_status;

/* Bytes of the static device scratch of fa_fwd_ex_noalloc (per GPU). */
#define FA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

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
 *          array (plus 1024 rows) below 2^31 bytes, and the launch grid
 *          (B*H*ceil(N/R) workgroups, where a workgroup takes R = 16 to 512
 *          query rows by dtype, d, mask and problem size) below 2^31.
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

/*
 * fa_fwd_ex -- the forward pass for decoding, grouped K/V heads and short
 * grids, with the work optionally split over key ranges.
 *
 * Same operation as fa_fwd, generalised in three ways:
 *   - queries and keys have their own lengths: q and o are [B, H, N_q, d],
 *     k and v are [B, H_kv, N_kv, d], lse is [B, H, N_q];
 *   - grouped heads: H_kv divides H and query head h reads K/V head
 *     h / (H / H_kv) (H_kv = H is ordinary multi-head attention, H_kv = 1
 *     shares one K/V head among all query heads).  The pages only name the
 *     technique, grouped-query attention, which maps a group of query heads
 *     onto one K/V head ("FlashAttention dissected", section "Interaction
 *     with the KV cache during inference");
 *   - causal masking is aligned to the end of the keys: key j is masked for
 *     query i when j > i + (N_kv - N_q), so that query row i stands at key
 *     position N_kv - N_q + i, as a decoding step that appends N_q tokens to
 *     a cache of N_kv keys does.  With N_q = N_kv this is fa_fwd's mask; a
 *     query with no visible key (possible when N_q > N_kv) gets O = 0 and
 *     LSE = -inf.
 * Split over keys (FlashDecoding, same section of "FlashAttention
 * dissected": with one query row the keys are split across compute units
 * to keep them busy): with num_splits > 1 the keys are cut into at most
 * num_splits ranges of equal length (a multiple of 64 keys; fewer ranges
 * when N_kv is short), every range is computed by its own workgroups into
 * an fp32 partial result plus its logsumexp in `workspace`, and a second
 * kernel merges the ranges exactly as fa_lse_combine does.  num_splits = 1
 * runs one kernel and needs no workspace (workspace may then be NULL).
 * fa_fwd_ex_default_splits gives a split count that fills the GPU.
 *
 * workspace        device memory of at least
 *                  fa_fwd_ex_workspace_bytes(B, H, N_q, N_kv, d, num_splits)
 *                  bytes, 16-byte aligned, owned by the caller and not
 *                  overlapping any other argument; its contents on entry do
 *                  not matter and are overwritten.  Two calls that share a
 *                  workspace must be ordered (same stream, or synchronised).
 * Everything else: as fa_fwd (validation before any launch, asynchronous on
 * `stream`, no allocation, no retained pointers).  Status: FA_ERR_SHAPE
 * also when H is not a multiple of H_kv (H_kv = 0 is allowed only with
 * H = 0); FA_ERR_WORKSPACE when num_splits < 1 or, for a split launch, the
 * workspace is NULL, smaller than required or misaligned.  N_kv = 0 is
 * valid: every row then has no visible key, and k and v may be NULL.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t d,
                    float scale, int causal, fa_dtype dtype, int64_t num_splits,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fa_fwd_ex_noalloc -- fa_fwd_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same operation, arguments, validation and results as
 * fa_fwd_ex with the same num_splits (bitwise: the same kernels run), minus
 * the workspace arguments: the split partials go to a static device array
 * of FA_NOALLOC_SCRATCH_BYTES (32 MiB) that every GPU the library runs on
 * holds from the first call until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 * The partials of a call need fa_fwd_ex_workspace_bytes(B, H, N_q, N_kv, d,
 * num_splits) bytes; more than FA_NOALLOC_SCRATCH_BYTES returns
 * FA_ERR_SCRATCH and launches nothing (use fewer splits, or fa_fwd_ex).  An
 * unsplit call (num_splits = 1, or keys too few to split) does not touch the
 * scratch.  The first split call on a device looks up that device's scratch
 * address once (hipGetSymbolAddress, with the device of `stream` current for
 * the lookup); FA_ERR_LAUNCH reports a failed lookup.
 *
 * Every call on one GPU shares that GPU's scratch: two split calls whose
 * kernels may overlap in time (different streams without ordering, or
 * different host threads) race on it and can corrupt each other's results.
 * Order such calls on one stream, or synchronise them.  Nothing needs to be
 * cleared between calls (each split writes all of its partials before the
 * merge reads them).
 */
fa_status fa_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv,
                            int64_t d, float scale, int causal, fa_dtype dtype,
                            int64_t num_splits, void* stream);

/* Workspace bytes fa_fwd_ex needs for `num_splits` (0 when the call runs
 * unsplit; -1 when the size overflows int64).  Invalid sizes give 0. */
int64_t fa_fwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t N_q, int64_t N_kv, int64_t d,
                                  int64_t num_splits);

/* A split count for fa_fwd_ex that gives MI355X's 256 compute units enough
 * workgroups when the unsplit grid is short (1 when it is already full or
 * the arguments are invalid): about one multi-wave bf16/fp16 workgroup or
 * two fp32 or one-wave workgroups per compute unit.  Small fp32 problems
 * with N_kv * d <= 65536 are not split: their unsplit kernel already spreads
 * 16-row blocks over the chip and is faster than a split call with its
 * combine step. */
int64_t fa_fwd_ex_default_splits(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                 int64_t d, int causal, fa_dtype dtype);

/*
 * fa_lse_combine -- merge attention results computed over disjoint key
 * ranges (the split-KV partials above, or the per-device results of a
 * sequence sharded across GPUs).
 *
 * o_part    device fp32 [splits, rows, d]: range s's output for each row,
 *           already divided by that range's own sum of exponentials
 *           (0 for a row with no visible key in the range).
 * lse_part  device fp32 [splits, rows]: range s's natural-log logsumexp
 *           (-inf for a row with no visible key in the range).
 * o         device [rows, d] of `dtype`, written in full:
 *           O = sum_s exp(LSE_s - LSE) O_s with LSE = log sum_s exp(LSE_s),
 *           the online-softmax rescaling of "FlashAttention dissected",
 *           section "The mathematical breakthrough: Tiling and Online
 *           Softmax", applied to whole ranges; a row with every LSE_s = -inf
 *           gets O = 0.
 * lse       device fp32 [rows] written in full (-inf for such rows), or NULL.
 * d         64 or 128.
 * Ownership, ordering and validation as fa_fwd: o_part and lse_part are only
 * read and must not overlap o or lse; o_part and o 16-byte aligned.
 */
fa_status fa_lse_combine(const float* o_part, const float* lse_part, int64_t splits,
                         int64_t rows, int64_t d, void* o, float* lse, fa_dtype dtype,
                         void* stream);

/*
 * fa_bwd -- gradients of the forward pass: given dO = dL/dO for
 * O = softmax(Q K^T * scale) V, computes dQ, dK, dV.
 *
 * The attention weights are not stored by fa_fwd; they are recomputed from
 * q, k and the forward pass's `lse` ("FlashAttention dissected", section
 * "Memory complexity: from O(N^2) to O(N)": the backward pass recomputes
 * what it needs from Q, K, V and the saved softmax statistics).  With
 * P_ij = exp(scale q_i.k_j - LSE_i) on the visible keys:
 *     D_i = dO_i . O_i,   dS_ij = P_ij (dO_i . v_j - D_i),
 *     dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,
 *     dQ_i = scale sum_j dS_ij k_j.
 *
 * q, k, v, o   the forward call's inputs and output: device, contiguous
 *              [B, H, N, d] of `dtype` (FA_F32, FA_BF16 or FA_F16), read
 *              only.  fp32 runs on fp32 MFMA with fp32 weights; bf16/fp16
 *              round P and dS to the input type as MFMA operands.
 * dout         device [B, H, N, d] of `dtype`: dL/dO, read only.
 * lse          device fp32 [B, H, N]: the lse fa_fwd wrote for the same
 *              q, k, v, scale and causal flag, read only.
 * dq, dk, dv   device [B, H, N, d] of `dtype`, written in full (rounded to
 *              nearest-even from fp32 accumulators).
 * delta        device fp32 [B, H, N], caller-owned scratch: overwritten with
 *              D_i = dO_i . O_i (the row dot products the gradients use).
 * B, H, N, d, scale, causal: as fa_fwd.
 * Buffers: 16-byte aligned (lse and delta 4-byte); outputs and delta may
 * not overlap each other or any input.  Runs three kernels on `stream`
 * (row dot products, then dK/dV, then dQ); no atomics, so results are
 * bitwise reproducible.  Validation, ordering and ownership as fa_fwd.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B,
                 int64_t H, int64_t N, int64_t d, float scale, int causal, fa_dtype dtype,
                 void* stream);

/*
 * fa_bwd_ex -- fa_bwd for grouped K/V heads and separate query and key
 * lengths: the gradients of fa_fwd_ex (any num_splits; the split only changes
 * how the forward computed O and LSE).
 *
 * q, o, dout, dq   device [B, H, N_q, d] of `dtype` (dq written in full).
 * k, v, dk, dv     device [B, H_kv, N_kv, d] of `dtype` (dk, dv written in
 *                  full); H_kv divides H and query head h uses K/V head
 *                  h / (H / H_kv), as in fa_fwd_ex.
 * lse, delta       device fp32 [B, H, N_q]: fa_fwd_ex's lse; caller-owned
 *                  scratch for the row dot products.
 * causal           the mask of fa_fwd_ex: key j is visible to query row i
 *                  when j <= i + N_kv - N_q.
 * Every query head of a group contributes to its K/V head: dK and dV are the
 * sums of the per-query-head gradients (chain rule through the shared K/V
 * head).  With num_splits = 1 one workgroup per (K/V head, 128 keys) forms
 * the whole sum in registers.  With num_splits > 1 the group's query heads
 * are cut into min(num_splits, H / H_kv) contiguous parts of near-equal
 * size; each part's workgroups write fp32 partial sums to `workspace` and a
 * second kernel adds the parts in part order, so the grid is larger (this
 * evens out the causal mask's uneven work per key tile) and results stay
 * bitwise reproducible for a given num_splits.  fa_bwd_ex_default_splits
 * gives a count suited to 256 compute units.  A query row that sees no key
 * gets a zero dQ row; with N_q = 0, dk and dv are zero-filled; with
 * N_kv = 0, dq is zero-filled.  Pointers of an empty side (q, o, dout, lse,
 * dq, delta when N_q = 0; k, v, dk, dv when N_kv = 0) may be NULL.
 *
 * workspace        device memory of at least
 *                  fa_bwd_ex_workspace_bytes(B, H, H_kv, N_q, N_kv, d,
 *                  num_splits) bytes, 16-byte aligned, caller-owned, not
 *                  overlapping any other argument; contents on entry do not
 *                  matter.  May be NULL when that size is 0 (one part).  Two
 *                  calls that share a workspace must be ordered.
 * Validation and alignment as fa_bwd, plus FA_ERR_SHAPE when H_kv does not
 * divide H, FA_ERR_WORKSPACE when num_splits < 1 or, with more than one
 * part, the workspace is NULL, short or misaligned, and FA_ERR_ALIAS when it
 * overlaps another argument.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B,
                    int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t d, float scale,
                    int causal, fa_dtype dtype, int64_t num_splits, void* workspace,
                    int64_t workspace_bytes, void* stream);

/* Workspace bytes fa_bwd_ex needs for `num_splits` head parts:
 * 2 * parts * B * H_kv * N_kv * d * 4 with parts = min(num_splits, H / H_kv),
 * 0 when the call runs in one part (num_splits <= 1, H = H_kv, N_q = 0 or
 * N_kv = 0) or the sizes are invalid, -1 when the size overflows int64. */
int64_t fa_bwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                  int64_t d, int64_t num_splits);

/* A head-part count for fa_bwd_ex: 1 without grouped heads or when the
 * unsplit dK/dV grid already holds enough workgroups for MI355X's 256
 * compute units (two per workgroup slot without a mask, four under the
 * causal mask, whose work per key tile is uneven); otherwise the smallest
 * divisor of H / H_kv that reaches that (parts of equal size), at most
 * H / H_kv (1 when the arguments are invalid). */
int64_t fa_bwd_ex_default_splits(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv,
                                 int64_t d, int causal, fa_dtype dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(fa_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
