/*
 * fa.h -- C ABI of the exact tiled attention forward library (libfa.so, gfx950).
 *
 * The operation. For every batch b, query head h and query position i:
 *     s_ij   = scale * <q_i, k_j>                       (j over the visible keys)
 *     O_i    = sum_j softmax_j(s_i.) v_j
 *     lse_i  = ln sum_j exp(s_ij)
 * This is standard attention as defined on the page "FlashAttention: The Algorithm
 * That Made Long-Context AI Possible" (section "The quadratic bottleneck in standard
 * attention"), computed the I/O-aware way described in the abstract of "FlashAttention:
 * Fast and Memory-Efficient Exact Attention with IO-Awareness" and the section "What
 * tiling changes" of the first page: key/value tiles stream through on-chip memory, a
 * running row maximum and running exponential sum replace the full softmax, and the
 * N x N score matrix never reaches device memory. The work is split over workgroups
 * per (batch, head, query tile) and, inside a workgroup, per wavefront over disjoint
 * query rows, as in the abstract of "FlashAttention-2: Faster Attention with Better
 * Parallelism and Work Partitioning" (items 2 and 3). The pages leave the following
 * open; the library takes these readings:
 *   - `scale` multiplies the scores before the softmax;
 *   - causal masking keeps key j for query i iff j <= i (square, no offset);
 *   - a key window (fa_fwd_local) keeps i - left <= j <= i + right on top of that;
 *   - grouped-query attention: query head h reads key/value head h / (H / Hkv);
 *   - lse is the natural log of the softmax denominator over the scaled scores;
 *   - e4m3 inputs (the low-precision mode in the abstract of "FlashAttention-3: Fast
 *     and Accurate Attention with Asynchrony and Low-precision") carry one descale per
 *     tensor: the logical value of an element is its e4m3 value times the descale.
 *
 * Layouts (row-major, contiguous, element strides implied by the shape):
 *     q, o : [B][N][H][d]        k, v : [B][N][Hkv][d]        lse : [B][H][N] float32
 * Element types: F16 -> q, k, v, o are IEEE binary16; BF16 -> bfloat16; FP8_E4M3 ->
 * q, k, v are OCP E4M3 ("fn", max 448) and o is bfloat16. Accumulation is float32.
 *
 * Ownership and execution. The caller owns every buffer (device memory). The library
 * allocates nothing, frees nothing and never synchronises: fa_fwd validates its
 * arguments on the host, enqueues one kernel on `stream` (a hipStream_t; NULL is the
 * null stream) and returns. A fault inside the kernel surfaces at the caller's next
 * synchronisation. q, k, v are only read; o and lse are fully overwritten; o and lse
 * must not overlap q, k, v or each other. No workspace is needed: memory use is linear
 * in N. The library keeps no state and may be called from several threads.
 *
 * Environment (read once, on first use):
 *   FA_LOG=1                    every launch prints "fa: <kernel> [<template arguments>]
 *                               grid <workgroups> block <threads>" to stderr;
 *   FA_FORCE_VARIANT=fp8_block_qk=bf16 | fp8_block_qk=e4m3
 *                               overrides the qk_e4m3 argument of fa_fwd_fp8_block after
 *                               its validation (for A/B runs of the two Q K^T paths).
 *
 * Errors. Every precondition is checked on the host before any HIP call; on error
 * nothing is enqueued and the outputs are untouched.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad flag, bad scale */
  FA_ERR_UNSUPPORTED = 2,   /* valid request the kernels do not implement (e.g. d) */
  FA_ERR_LAUNCH = 3,        /* the HIP runtime rejected the launch */
  FA_ERR_SCRATCH = 4        /* the request needs more than the library's static scratch */
} fa_status;

typedef enum {
  FA_DTYPE_F16 = 0,
  FA_DTYPE_BF16 = 1,
  FA_DTYPE_FP8_E4M3 = 2
} fa_dtype;

/*
 * Attention forward.
 *   q, k, v   device pointers, layouts above, 16-byte aligned.
 *   o         device pointer, [B][N][H][d] of the output type, 16-byte aligned.
 *   lse       device pointer, [B][H][N] float32, 4-byte aligned.
 *   B, H, Hkv, N, d   sizes: B >= 1, N >= 1, 1 <= Hkv <= H, H % Hkv == 0,
 *             d in {64, 128}; every tensor must have fewer than 2^31 elements, and K (and
 *             V) of one batch fewer than 2^31 bytes (else FA_ERR_UNSUPPORTED).
 *   causal    0 (no mask) or 1 (key j visible to query i iff j <= i).
 *   scale     finite, > 0; multiplies q.k before the softmax (1/sqrt(d) is usual).
 *   dtype     element type of q, k, v (see above).
 *   descale_qkv  FP8_E4M3 only: host pointer to three finite, positive floats
 *             (descale of q, k, v); must be NULL for the other types.
 *   stream    hipStream_t to enqueue on (NULL = null stream).
 * Returns FA_OK once the kernel is enqueued.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int N, int d, int causal, float scale,
                 fa_dtype dtype, const float* descale_qkv, void* stream);

/*
 * Attention forward with a key window (sliding-window / local attention). The page
 * "FlashAttention: The Algorithm That Made Long-Context AI Possible" names
 * sliding-window patterns (section "Why context lengths exploded after 2022") without
 * defining them; the library's reading: key j is visible to query i iff
 *     i - window_left <= j <= i + window_right,
 * intersected with the causal mask when causal = 1. A negative bound (or one >= N)
 * leaves that side unbounded, so (-1, -1) is fa_fwd itself and (-1, 0) without the
 * causal flag is the causal mask. Every query sees at least its own key, so no row is
 * empty. The kernel visits only the key tiles inside the band of each query tile: the
 * work is linear in N for a fixed window. Every other argument, layout, ownership rule
 * and error is as for fa_fwd (window bounds themselves are never an error).
 */
fa_status fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, int causal, int window_left,
                       int window_right, float scale, fa_dtype dtype,
                       const float* descale_qkv, void* stream);

/* Queries and keys per block of a block-sparse mask. */
#define FA_SPARSE_BLOCK 64

/*
 * Block-sparse attention: the block-sparse variant named in the abstract of
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness", which
 * the pages do not define further. The library's reading: `block_mask` is a device
 * buffer of [mask_heads][nb][nb] bytes, nb = ceil(N / FA_SPARSE_BLOCK), row-major; key j
 * is visible to query i of head h iff
 *     block_mask[hm][i / FA_SPARSE_BLOCK][j / FA_SPARSE_BLOCK] != 0,
 * hm = 0 when mask_heads = 1 (one mask for every head) and hm = h when mask_heads = H;
 * causal = 1 further keeps only j <= i. Attention over the visible keys is exact. A
 * query with no visible key has no softmax: its output row is 0 and its lse is -inf.
 * The kernel visits, per query tile, only the key blocks that some query of the tile
 * keeps, so the work scales with the number of kept blocks.
 * F16 and BF16 only (FP8_E4M3 is FA_ERR_UNSUPPORTED); N <= 131072 (FA_ERR_UNSUPPORTED
 * beyond); mask_heads must be 1 or H and block_mask non-null (else
 * FA_ERR_INVALID_ARG). The mask is only read. Every other argument, layout, ownership
 * rule and error is as for fa_fwd.
 */
fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Hkv, int N, int d, int causal,
                              const unsigned char* block_mask, int mask_heads, float scale,
                              fa_dtype dtype, void* stream);

/* Rows (sequence positions) per block of the e4m3 block quantisation. */
#define FA_FP8_BLOCK_ROWS 64

/*
 * Block quantisation to e4m3 with optional incoherent processing: the two parts of the
 * FP8 mode named in the abstract of "FlashAttention-3: Fast and Accurate Attention with
 * Asynchrony and Low-precision", which defines neither; the library's reading:
 *   - x is a [B][N][Hx][d] tensor of in_dtype (F16 or BF16), 16-byte aligned;
 *   - if `signs` is not NULL (device pointer to d floats, each +1 or -1, 16-byte
 *     aligned), every row is first replaced by (x * signs) H, H the d x d
 *     Sylvester-Hadamard matrix (entries +-1, H H^T = d I), computed in float32 by the
 *     fast Walsh-Hadamard butterflies h = 1, 2, ..., d/2; rotating both Q and K this way
 *     multiplies every score by d, so pass scale / d to the attention call;
 *   - every block of FA_FP8_BLOCK_ROWS consecutive positions of one (b, head) gets the
 *     scale 2^e, e the smallest integer with (block max |x|) * 2^-e <= 448, floored at
 *     -127, and 0 for an all-zero block; scales[(b * Hx + head) * nb + blk] = e + 127
 *     (an E8M0 byte), nb = ceil(N / FA_FP8_BLOCK_ROWS);
 *   - codes (same layout as x, one byte each, 8-byte aligned) are the OCP E4M3 round-to-
 *     nearest-even of x * 2^-e (exact scaling, saturated at +-448).
 * Inputs must be finite. d in {64, 128}. Ownership, errors and execution as for fa_fwd
 * (F16/BF16 only: FP8_E4M3 input is FA_ERR_UNSUPPORTED). One kernel on `stream`.
 */
fa_status fa_quantize_e4m3_block(const void* x, fa_dtype in_dtype, int B, int N, int Hx, int d,
                                 const float* signs, void* codes, unsigned char* scales,
                                 void* stream);

/*
 * Attention forward on block-quantised e4m3 inputs (as written by
 * fa_quantize_e4m3_block): the logical value of element (b, n, head, t) is its e4m3 code
 * times 2^(scale byte - 127) of block n / FA_FP8_BLOCK_ROWS of that (b, head).
 *   q_scales  device pointer, [B][H][nb] bytes; k_scales, v_scales [B][Hkv][nb] bytes,
 *             nb = ceil(N / FA_FP8_BLOCK_ROWS).
 *   qk_e4m3   0: Q K^T runs on the bf16 MFMA after an exact widening of the codes (times
 *             their block scales); exact products, float32 sums, for any codes.
 *             1: Q K^T runs on the e4m3 MFMA with the Q and K block scales as its scale
 *             operands (about 1.2x faster). That unit sums each 64-term product with
 *             limited internal precision, so a score moves by an amount that grows with
 *             the largest products of its row: fine after incoherent processing (Q and K
 *             rotated by fa_quantize_e4m3_block with signs, which spreads outliers), not
 *             on raw codes with outliers. Any other value is FA_ERR_INVALID_ARG.
 * V scales are the per-tile scale operand of the scaled e4m3 P.V MFMA. o is bfloat16.
 * N <= 131072 (FA_ERR_UNSUPPORTED beyond). Otherwise as fa_fwd with dtype FP8_E4M3 (no
 * descale argument; when Q and K were rotated by the quantiser, pass scale / d).
 */
fa_status fa_fwd_fp8_block(const void* q, const void* k, const void* v,
                           const unsigned char* q_scales, const unsigned char* k_scales,
                           const unsigned char* v_scales, void* o, float* lse, int B, int H,
                           int Hkv, int N, int d, int causal, float scale, int qk_e4m3,
                           void* stream);

/*
 * Gradient of the attention forward (fa_fwd) for an upstream gradient dout of o. The
 * pages report training speed-ups but print no backward algorithm; the library computes
 * the analytic gradient of the forward definition, with no gradient through lse:
 *     D_i = <dout_i, o_i>,  P_ij = exp(scale <q_i, k_j> - lse_i)  (0 where masked)
 *     dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (<dout_i, v_j> - D_i)
 *     dk_j = scale sum_i dS_ij q_i,  dq_i = scale sum_j dS_ij k_j
 * summing dk and dv over the query heads of each key/value head (grouped-query).
 *   q, k, v     the forward's inputs; o and lse its outputs (lse as written by fa_fwd);
 *   dout        [B][N][H][d], the gradient of o;
 *   dq          [B][N][H][d]; dk, dv [B][N][Hkv][d]; outputs, fully overwritten;
 *   q..dv       device pointers, 16-byte aligned, of dtype F16 or BF16 (FP8_E4M3 is
 *               FA_ERR_UNSUPPORTED); lse 4-byte aligned float32;
 *   workspace   device scratch of at least fa_bwd_workspace_bytes(B, H, N) bytes, 4-byte
 *               aligned, owned by the caller; it holds D between the launches of one call
 *               (calls that share a workspace must not overlap);
 *   causal      0 or 1 (key windows are not supported here); scale as for fa_fwd.
 * Enqueues three kernels on `stream` (D, then dk/dv, then dq) and returns. Accumulation
 * is float32; dq, dk, dv are rounded once. Deterministic (no atomics). Errors as for
 * fa_fwd; every check happens on the host before any launch.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, fa_dtype dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Split-KV attention forward for decode: Nq queries that are the last Nq positions of a
 * sequence whose keys and values cover all Nk positions (Nq <= Nk). Under the causal mask
 * query i sees keys j <= Nk - Nq + i (with Nq = Nk this is fa_fwd's mask). The pages name
 * work-centric and split schedules for decoding (the Lean Attention and Stream-K titles
 * of their reference lists) without describing them; the library's reading: the key axis
 * of each (batch, key/value head) is cut into ranges processed independently, each
 * leaving an output normalised over its keys and its log-sum-exp, merged exactly by
 * lse = ln sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
 *   q, o       [B][Nq][H][d]; k, v [B][Nk][Hkv][d]; lse [B][H][Nq] float32;
 *   num_splits ranges per (batch, key/value head); <= 0 picks a count that keeps the GPU
 *              busy; the effective count is at most ceil(Nk / 32);
 *   workspace  device scratch of at least fa_fwd_splitkv_workspace_bytes(...) bytes (same
 *              num_splits), 16-byte aligned, owned by the caller (partial outputs);
 *              calls sharing a workspace must not overlap.
 * Requires (H / Hkv) * Nq <= 64 (query rows sharing one key/value head); otherwise
 * FA_ERR_UNSUPPORTED (use fa_fwd). q, k, v 16-byte aligned, o and lse 4-byte aligned;
 * dtype F16 or BF16; d in {64, 128}. Enqueues two kernels (partials, merge) on `stream`.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int num_splits);
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         fa_dtype dtype, int num_splits, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments (minus workspace and workspace_bytes), semantics, kernels and
 * results as fa_fwd_splitkv with the same num_splits. The partial outputs go to a scratch
 * array of FA_SPLITKV_STATIC_SCRATCH_BYTES bytes that the library holds on each GPU it
 * runs on until the process ends; requests whose fa_fwd_splitkv_workspace_bytes exceeds
 * that size return FA_ERR_SCRATCH (use fa_fwd_splitkv with a caller workspace). The call
 * allocates nothing. Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (concurrent streams, or threads) race and must be serialised by the caller.
 * Nothing in the array needs to start at zero: each call writes every partial it reads.
 * The array's device address is looked up on a device's first call (FA_ERR_LAUNCH if the
 * lookup fails).
 */
#define FA_SPLITKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                                fa_dtype dtype, int num_splits, void* stream);

/*
 * Shape query: byte sizes of every buffer fa_fwd reads or writes for these arguments,
 * after the same size checks fa_fwd makes. Any output pointer may be NULL.
 * workspace_bytes is always 0 (no scratch memory). Pure host function.
 */
fa_status fa_fwd_query(int B, int H, int Hkv, int N, int d, int causal, fa_dtype dtype,
                       size_t* q_bytes, size_t* kv_bytes, size_t* o_bytes, size_t* lse_bytes,
                       size_t* workspace_bytes);

/* Static, human-readable text for a status code. */
const char* fa_status_string(fa_status s);

/* Library version, encoded as major * 10000 + minor * 100 + patch (10300: fa_fwd_splitkv_static). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
