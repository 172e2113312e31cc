/*
 * bi_logprob.h - batch-invariant per-token logprob, entropy and gradient over a
 * large vocabulary, for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For row i of a logits matrix z [n_rows, vocab] (bf16 or
 * fp32, -inf allowed for masked columns), its label y_i and an optional weight
 * w_i, with m = max_j z_j and F = { j : z_j > -inf }:
 *
 *   lse      = m + ln sum_{j in F} exp(z_j - m)
 *   logprob  = z_y - lse                    (+0.0 when y == ignore_index)
 *   entropy  = lse - sum_{j in F} p_j z_j = -sum_{j in F} p_j ln p_j
 *   grad_j   = w * (p_j - [j == y]),   p_j = exp(z_j - lse)
 *
 * Sources (page titles and sections):
 *  - "[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan PR
 *    #4685), Summary and Why: token logprobs and entropy from per-token
 *    sufficient statistics (global maximum, softmax denominator, target
 *    contribution, entropy-weighted sum); entropy is a metric without a
 *    gradient; the per-token gradient comes from the cross-entropy backward.
 *  - same page, Correctness and compatibility: ignored labels, partially
 *    masked logits, non-uniformly weighted gradients, FP32/BF16, even and
 *    uneven vocabulary sizes.
 *  - same page, review reply "Input sharding contract of compute_logprobs":
 *    full-row calls take [N, V] logits; the vocabulary-parallel path takes the
 *    local shard [T, V_local] and needs the global vocabulary size.
 *  - same page, review reply "Batch invariance under the patched logprob
 *    path", Q1/Q2: a trainer and a generator agree bit for bit only when they
 *    use the same operation sequence and summation grouping; the maximum
 *    combines exactly across shards, sums do not.
 *  - "torchtitan-batch-invarient-GDN" (README), intro and Result: the goal is
 *    the trainer's recomputed logprob matching the generator's bit for bit.
 *
 * Batch invariance.  Each row is reduced by one workgroup whose size, vector
 * width, column-to-lane map and reduction tree are functions of (dtype, width)
 * only - never of n_rows, the grid, the device or the row's alignment.  Every
 * row's outputs are therefore bit-identical whatever batch it sits in.  The
 * chunked path (bi_vocab_chunk_stats + bi_stats_combine) is exact in real
 * arithmetic but is NOT bitwise equal to bi_logprob_fwd; callers that need
 * trainer/generator bit equality use bi_logprob_fwd on full rows.
 *
 * Conventions for every entry point.
 *  - Array arguments are DEVICE pointers; the caller owns every buffer and
 *    keeps it alive until the work queued on `stream` has finished.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  They never synchronize and never allocate.
 *  - Arguments are validated on the host before anything is queued; on any
 *    error nothing is launched and a bi_status code is returned.  The reason
 *    is also kept, per thread, for bi_last_error().
 *  - Logits are row-major with a row pitch of `row_stride` elements
 *    (row_stride >= width); the last dimension is contiguous.  Pointers must be
 *    aligned to their element size; rows need not be 16-byte aligned.
 *  - Labels are int64.  A label that is neither ignore_index nor in
 *    [0, vocab) cannot be checked on the host without a sync: the kernels OR
 *    BI_FLAG_BAD_LABEL into *status_flag (when non-NULL) and write NaN for that
 *    row's logprob and gradient row.
 *  - logprob, entropy and lse are always fp32.
 */
#ifndef BI_LOGPROB_H
#define BI_LOGPROB_H

#include <stdint.h>

#if defined(__GNUC__)
#define BI_API __attribute__((visibility("default")))
#else
#define BI_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of logits and gradients. */
enum { BI_F32 = 0, BI_BF16 = 1 };

/* Status codes returned by every entry point. */
enum {
  BI_OK = 0,
  BI_ERR_NULL = 1,   /* a required pointer is NULL */
  BI_ERR_SHAPE = 2,  /* bad size, stride, vocabulary size or offset */
  BI_ERR_DTYPE = 3,  /* unknown dtype or unsupported (logits, grad) pair */
  BI_ERR_ALIGN = 4,  /* a pointer is not aligned to its element size */
  BI_ERR_LAUNCH = 5  /* the HIP launch failed (see bi_last_error) */
};

/* Bits ORed into *status_flag by the kernels. */
enum { BI_FLAG_BAD_LABEL = 1 };

typedef void* bi_stream_t; /* a hipStream_t */

/* Per-(chunk, row) sufficient statistics, 16 bytes.
 *   max          m_c = max of the chunk's logits (-inf if all are -inf)
 *   sumexp       S_c = sum over finite columns of exp(z - m_c)
 *   target       z_y if the label lies in this chunk, else 0.0 (NaN for a bad
 *                label), so that summing over chunks yields z_y
 *   sumexp_logit U_c = sum over finite columns of exp(z - m_c) * (z - m_c);
 *                the unshifted sum of exp(z - m_c) * z is U_c + m_c * S_c
 * A fully masked chunk has (max, sumexp, sumexp_logit) = (-inf, 0, 0). */
typedef struct {
  float max;
  float sumexp;
  float target;
  float sumexp_logit;
} bi_stats;

/* Forward over full rows: logprob, entropy and lse per row.
 * Defined in PR #4685 (Summary, Why) and its reply "Input sharding contract of
 * compute_logprobs" (full [N, V] logits; logprob = -cross_entropy, reduction
 * "none").  This is the batch-invariant path.
 *   logits       [n_rows, row_stride] of dtype (BI_F32 or BI_BF16); columns
 *                [0, vocab) are read
 *   n_rows       >= 0; 0 is a no-op
 *   vocab        1 <= vocab < 2^29
 *   row_stride   >= vocab, in elements
 *   labels       [n_rows] int64
 *   ignore_index label value of ignored rows (-100 in the pages' setting);
 *                such rows get logprob +0.0 and still get entropy and lse
 *   logprob, entropy, lse  [n_rows] fp32 each; any may be NULL, not all
 *   status_flag  optional device int32, see BI_FLAG_BAD_LABEL
 */
BI_API int bi_logprob_fwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                   int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                   float* logprob, float* entropy, float* lse,
                   int32_t* status_flag, bi_stream_t stream);

/* Backward: grad = w * (softmax - onehot(label)) from the saved lse.
 * Defined in PR #4685 (Summary: reuse the cross-entropy backward for
 * per-token gradients; Correctness and compatibility: non-uniformly weighted
 * gradients; the review's backward returns only the logits gradient).
 *   lse          [n_rows] fp32, from bi_logprob_fwd or bi_stats_combine
 *   weights      [n_rows] fp32 per-token weights, NULL means 1.  For a loss
 *                L = sum_i w_i * CE_i = -sum_i w_i * logprob_i, pass
 *                w_i = -dL/dlogprob_i.
 *   grad         [n_rows, grad_row_stride] of grad_dtype; columns [0, vocab)
 *                are written.  Ignored rows are written +0.0 without reading
 *                their logits.  Masked (-inf) columns get +0.0.
 *   (dtype, grad_dtype) must be (F32, F32), (BF16, BF16) or (BF16, F32);
 *   a bf16 gradient is the fp32 value rounded to nearest even.
 *   grad_row_stride >= vocab.
 * Elementwise given lse: each element's bits depend only on its logit and its
 * row's lse, weight and label, however the rows are split over workgroups.
 */
BI_API int bi_logprob_bwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                   int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                   const float* lse, const float* weights,
                   void* grad, int grad_dtype, int64_t grad_row_stride,
                   int32_t* status_flag, bi_stream_t stream);

/* Forward and backward in one pass over each row, for callers that know the
 * per-token weight before the forward: logprob, entropy, lse and the gradient
 * w * (softmax - onehot), reading the logits once.  Every output is bit-
 * identical to bi_logprob_fwd followed by bi_logprob_bwd with the same
 * weights (same lane map, reduction tree and per-element arithmetic).
 * Defined as the composition of the two calls above (PR #4685, Summary and
 * Why; Correctness and compatibility for the weights).
 *   weights      [n_rows] fp32, NULL means 1 (as in bi_logprob_bwd)
 *   logprob, entropy, lse  [n_rows] fp32 each; each may be NULL
 *   grad         required; layout and dtype rules as in bi_logprob_bwd.  Its
 *                byte range must not overlap the logits' (BI_ERR_SHAPE):
 *                rows' gradients are written while other rows are still
 *                to be read.
 */
BI_API int bi_logprob_fwd_bwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                              int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                              const float* weights, float* logprob, float* entropy, float* lse,
                              void* grad, int grad_dtype, int64_t grad_row_stride,
                              int32_t* status_flag, bi_stream_t stream);

/* The same single pass, with the per-token weight derived in the kernel from
 * the logprob it has just computed: the clipped-ratio policy-gradient
 * surrogate of DAPO/GRPO-style losses ("torchtitan-batch-invarient-GDN",
 * MATH recipe: DAPO with clip (0.2, 0.28); PR #4685, Summary: per-token
 * gradients for DAPO/GRPO losses).  Per token, with r = exp(logprob -
 * old_logprob), advantage A and scale c:
 *   loss   = -c * min(r A, clip(r, 1 - clip_low, 1 + clip_high) A)
 *   weight = -d loss / d logprob = c A r if the unclipped term is the minimum
 *            (ties count as unclipped), else 0
 *   grad   = weight * (softmax - onehot)  = d loss / d logits
 * Ignored tokens have loss 0, weight 0 and a zero gradient row.  logprob,
 * entropy and lse are bit-identical to bi_logprob_fwd, and the gradient to
 * bi_logprob_bwd given the written weights.
 *   old_logprob, advantages  [n_rows] fp32, required (the behaviour policy's
 *                logprob of the label and the token's advantage)
 *   loss_scale   [n_rows] fp32, NULL means 1 (e.g. 1 / number of tokens)
 *   clip_low     in [0, 1); clip_high >= 0
 *   loss, weight [n_rows] fp32 outputs, each may be NULL
 *   grad         as in bi_logprob_fwd_bwd (not overlapping the logits)
 */
BI_API int bi_policy_loss_fwd_bwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                                  int64_t row_stride, const int64_t* labels,
                                  int64_t ignore_index, const float* old_logprob,
                                  const float* advantages, const float* loss_scale,
                                  float clip_low, float clip_high, float* logprob,
                                  float* entropy, float* lse, float* loss, float* weight,
                                  void* grad, int grad_dtype, int64_t grad_row_stride,
                                  int32_t* status_flag, bi_stream_t stream);

/* Statistics of one vocabulary chunk: global columns
 * [vocab_offset, vocab_offset + chunk_width) held as a [n_rows, chunk_width]
 * view.  Defined in PR #4685, Why (shard-local sufficient statistics) and the
 * reply "Input sharding contract of compute_logprobs" (the vocabulary-parallel
 * path takes the local shard and requires the global vocabulary size; without
 * it the call fails).
 *   logits_chunk  points at global column vocab_offset of row 0
 *   chunk_width   >= 1; vocab_offset >= 0; vocab_offset + chunk_width <= vocab
 *   vocab         the global vocabulary size (labels are global columns)
 *   stats         [n_rows] bi_stats for this chunk
 */
BI_API int bi_vocab_chunk_stats(const void* logits_chunk, int dtype, int64_t n_rows,
                         int64_t chunk_width, int64_t row_stride,
                         int64_t vocab_offset, int64_t vocab,
                         const int64_t* labels, int64_t ignore_index,
                         bi_stats* stats, int32_t* status_flag, bi_stream_t stream);

/* Exact combine of chunk statistics, chunks taken in ascending order.
 * Defined in PR #4685, Why, and the reply "Batch invariance under the
 * patched logprob path", Q2: M = max_c m_c is exact; then, for c = 0, 1, ...,
 * S += e^(m_c - M) S_c, U += e^(m_c - M) (U_c + (m_c - M) S_c), t += t_c;
 * a chunk with S_c == 0 contributes nothing.  lse = M + ln S,
 * logprob = t - lse (+0.0 if ignored), entropy = ln S - U / S.
 *   stats    [n_chunks][n_rows] bi_stats (chunk-major)
 *   n_chunks >= 1
 *   logprob, entropy, lse  [n_rows] fp32 each; any may be NULL, not all
 */
BI_API int bi_stats_combine(const bi_stats* stats, int64_t n_chunks, int64_t n_rows,
                     const int64_t* labels, int64_t ignore_index,
                     float* logprob, float* entropy, float* lse, bi_stream_t stream);

/* Several token ids per row sharing one lse: the generator's
 * compute_logprobs(logits, labels) with multi-column token ids (PR #4685,
 * Correctness and compatibility).  lse and entropy are bit-identical to
 * bi_logprob_fwd, and so is every column whose label equals the row's label.
 *   labels       [n_rows, label_stride] int64; columns [0, k) are used
 *   k            >= 1 token ids per row
 *   logprob      [n_rows, k] fp32 (row-major, contiguous), required:
 *                z[y] - lse, +0.0 for ignore_index, NaN for a bad id
 *   entropy, lse [n_rows] fp32, each may be NULL
 */
BI_API int bi_logprob_fwd_multi(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                                int64_t row_stride, const int64_t* labels, int64_t label_stride,
                                int64_t k, int64_t ignore_index, float* logprob, float* entropy,
                                float* lse, int32_t* status_flag, bi_stream_t stream);

/* Trainer-vs-generator logprob difference metrics ("torchtitan-batch-
 * invarient-GDN", Code map and Result: bit_wise logprob_diff mean / abs_mean
 * / max and ratio_tokens_different).  With d = a - b over the tokens whose
 * label is not ignore_index (all tokens when labels is NULL):
 *   out[0] = mean d, out[1] = mean |d|, out[2] = max |d|,
 *   out[3] = fraction of tokens whose fp32 bit patterns differ.
 * Sums run in fp64 in a fixed order; no valid token gives zeros.
 *   a, b   [n] fp32 device vectors; labels [n] int64 or NULL; out [4] fp32
 */
BI_API int bi_logprob_diff_stats(const float* a, const float* b, const int64_t* labels,
                                 int64_t ignore_index, int64_t n, float* out,
                                 bi_stream_t stream);

/* lm_head projection fused with the chunk statistics: the logits
 * z[n, v] = sum_k hidden[n, k] * weight[v, k] of a block of lm_head rows are
 * computed on the matrix cores (bf16 inputs, fp32 accumulation) and reduced
 * straight to bi_stats per token, so the logits never reach memory (the
 * chunked lm_head of "ZeroSyncGRPOTrainer - #6949"; shard-local statistics,
 * PR #4685 Why).  Rows are cut into tiles of 256; tile c of token n is
 * written to stats[c * n_tokens + n], with the same meaning as
 * bi_vocab_chunk_stats on those 256 columns.  bi_stats_combine over the
 * bi_lmhead_tiles(n_vocab_rows) tiles then yields logprob, entropy and lse.
 * Each logit is the same MFMA sequence whatever n_tokens is (batch-
 * invariant).  The fp32 logits are used as computed (not rounded to bf16).
 *   hidden  [n_tokens, hidden_stride] bf16, 16-byte aligned rows
 *   weight  [n_vocab_rows, weight_stride] bf16 (the lm_head rows of global
 *           vocabulary ids vocab_offset .. vocab_offset + n_vocab_rows - 1)
 *   d       hidden size, a positive multiple of 64 (at most 2^22); strides
 *           multiples of 8, at most 2^22 elements
 *   stats   [bi_lmhead_tiles(n_vocab_rows)][n_tokens] bi_stats, 16-byte aligned
 */
BI_API int bi_lmhead_tile_stats(const void* hidden, const void* weight, int64_t n_tokens,
                                int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                                int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                                const int64_t* labels, int64_t ignore_index, bi_stats* stats,
                                int32_t* status_flag, bi_stream_t stream);

/* Number of tiles bi_lmhead_tile_stats writes for n_vocab_rows rows: tile t
 * covers rows t * bi_lmhead_tile_rows() .. (t + 1) * bi_lmhead_tile_rows() - 1
 * (the last one clipped). */
BI_API int64_t bi_lmhead_tiles(int64_t n_vocab_rows);

/* lm_head rows per statistics tile of bi_lmhead_tile_stats (256). */
BI_API int64_t bi_lmhead_tile_rows(void);

/* Gradient of the lm_head logits: G[v, n] = w_n * (softmax(z_n)[v] - [v == y_n])
 * for the rows of one vocabulary block, with z = hidden @ weight^T recomputed
 * on the matrix cores by the same MFMA sequence as bi_lmhead_tile_stats and
 * the lse from bi_stats_combine (the cross-entropy backward of PR #4685
 * Summary, on the lm_head logits; bi_logprob_bwd's arithmetic per element).
 *   lse            [n_tokens] fp32, the full-vocabulary lse of each token
 *   token_weights  [n_tokens] fp32 or NULL (= 1); ignored tokens get +0.0,
 *                  bad labels NaN (and BI_FLAG_BAD_LABEL)
 *   grad_logits    [n_vocab_rows, grad_stride] bf16, vocabulary-major (row v
 *                  holds the tokens), RNE; grad_stride >= n_tokens
 *   other arguments as for bi_lmhead_tile_stats */
BI_API int bi_lmhead_grad_logits(const void* hidden, const void* weight, int64_t n_tokens,
                                 int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                                 int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                                 const int64_t* labels, int64_t ignore_index, const float* lse,
                                 const float* token_weights, void* grad_logits,
                                 int64_t grad_stride, int32_t* status_flag, bi_stream_t stream);

/* lm_head backward from the saved lse: grad_hidden += G @ weight and
 * grad_weight = G^T @ hidden with G as in bi_lmhead_grad_logits (the chunked
 * lm_head backward of "ZeroSyncGRPOTrainer - #6949": bf16 GEMMs with fp32
 * accumulation).  The vocabulary block is processed in chunks of as many
 * rows (a multiple of 256) as the workspace holds: per chunk the grad-logits
 * kernel writes G (bf16, vocabulary-major, padded with zeros to whole 64-deep
 * K stages: rows to a multiple of 64, tokens to n_tokens rounded up to 64),
 * then G @ weight and G^T @ hidden run on the lm_head kernel's matrix-core
 * pipeline, reading G, the lm_head rows and the hidden states as they are
 * stored (transposing LDS reads where an operand is stored [K][columns]), all
 * on `stream`.  grad_weight rows are the same bits whatever the chunking;
 * grad_hidden sums the chunks in order (same bits for the same workspace size
 * on every run).
 *   grad_hidden    [n_tokens, grad_hidden_stride] fp32, ACCUMULATED (zero it
 *                  for a fresh gradient; vocabulary shards add their parts)
 *   grad_weight    [n_vocab_rows, grad_weight_stride] of grad_weight_dtype
 *                  (BI_F32 or BI_BF16), overwritten
 *   workspace      device memory, 256-byte aligned, of workspace_bytes >=
 *                  bi_lmhead_backward_workspace(n_tokens, d, chunk_rows) for
 *                  chunks of chunk_rows (at least one 256-row chunk of G); it
 *                  is in use until the queued work ends
 * n_tokens <= 2^22; other sizes and strides must fit in 32 bits, and d and
 * the strides follow bi_lmhead_tile_stats.  Nothing is allocated and nothing
 * synchronizes; calls on different streams with their own workspaces run
 * concurrently.  n_tokens == 0 or n_vocab_rows == 0 writes nothing. */
BI_API int bi_lmhead_backward(const void* hidden, const void* weight, int64_t n_tokens,
                              int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                              int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                              const int64_t* labels, int64_t ignore_index, const float* lse,
                              const float* token_weights, float* grad_hidden,
                              int64_t grad_hidden_stride, void* grad_weight,
                              int grad_weight_dtype, int64_t grad_weight_stride,
                              void* workspace, int64_t workspace_bytes, int32_t* status_flag,
                              bi_stream_t stream);

/* Size of the static device scratch of bi_lmhead_backward_noalloc (64 MiB on
 * every GPU the library runs on, held until the process ends) and the most
 * tokens it serves: one 256-row chunk of the logits gradient, bf16, with the
 * tokens rounded up to 64. */
#define BI_LMHEAD_NOALLOC_SCRATCH_BYTES (64 << 20)
#define BI_LMHEAD_NOALLOC_MAX_TOKENS 131072

/* bi_lmhead_backward without a workspace, for callers that cannot allocate
 * or pass device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, outputs and arithmetic as
 * bi_lmhead_backward, with G's chunks in a static device array of
 * BI_LMHEAD_NOALLOC_SCRATCH_BYTES instead of the caller's workspace: the
 * results are bit-identical to bi_lmhead_backward given a workspace of that
 * many bytes.  The array's device address is looked up once per device, on
 * the first call made with that device current.
 *   n_tokens  at most BI_LMHEAD_NOALLOC_MAX_TOKENS (131,072); more returns
 *             BI_ERR_SHAPE before anything is queued
 * Nothing is allocated (no hipMalloc, no library allocation).  Every call on
 * one GPU uses that GPU's one array: calls that may overlap on one GPU (on
 * different streams, or from host threads whose calls are not ordered on one
 * stream) race and give wrong results; calls queued on one stream are
 * ordered and safe.  Nothing in the array needs to start at zero: each chunk
 * writes every element of G that its products read. */
BI_API int bi_lmhead_backward_noalloc(const void* hidden, const void* weight, int64_t n_tokens,
                                      int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                                      int64_t weight_stride, int64_t vocab_offset,
                                      int64_t vocab, const int64_t* labels,
                                      int64_t ignore_index, const float* lse,
                                      const float* token_weights, float* grad_hidden,
                                      int64_t grad_hidden_stride, void* grad_weight,
                                      int grad_weight_dtype, int64_t grad_weight_stride,
                                      int32_t* status_flag, bi_stream_t stream);

/* Workspace bytes for bi_lmhead_backward with chunks of chunk_rows lm_head
 * rows (rounded up to a multiple of 256): one chunk of G, its rows by
 * n_tokens rounded up to 64, in bf16; -1 for bad arguments (negative sizes,
 * chunk_rows < 1, n_tokens > 2^22).  d is validated only. */
BI_API int64_t bi_lmhead_backward_workspace(int64_t n_tokens, int64_t d, int64_t chunk_rows);

/* Human-readable name of a status code (static string). */
BI_API const char* bi_status_string(int status);

/* Detail of the last error returned on this thread ("" if none). */
BI_API const char* bi_last_error(void);

/* The launch geometry used for rows of `width` columns of `dtype`: threads per
 * workgroup, elements per 128-bit load and loads per rescale group.  It is a
 * function of (dtype, width) only; this is the batch-invariance contract. */
BI_API int bi_row_geometry(int dtype, int64_t width, int* threads, int* elems_per_load,
                    int* loads_per_group);

#ifdef __cplusplus
}
#endif

#endif /* BI_LOGPROB_H */
