// bi_lmhead_bwd.hip - the lm_head backward: gradients of the hidden states and
// of the lm_head rows from the saved lse, without the [N, V] logits or their
// gradient ever existing in full.  C ABI: bi_lmhead_backward,
// bi_lmhead_backward_noalloc, bi_lmhead_backward_workspace
// (include/bi_logprob.h).
//
// What is computed: with G[n, v] = w_n * (softmax(z_n)[v] - [v == y_n]) the
// cross-entropy backward of "[RL] Avoid full-vocab gather for TP policy
// statistics" (torchtitan PR #4685, Summary) on the lm_head logits
// z = hidden @ weight^T, the chain rule gives grad_hidden = G @ weight and
// grad_weight = G^T @ hidden: the chunked lm_head backward of
// "ZeroSyncGRPOTrainer" (bf16 GEMMs with fp32 accumulation).
//
// How: the vocabulary shard is cut into chunks of rows that fit the caller's
// workspace.  For each chunk, the grad-logits kernel recomputes its logits on
// the matrix cores (the forward's exact MFMA sequence) and writes G for the
// chunk as bf16, vocabulary-major [rows][ldg], padded with zeros to whole
// 64-deep K stages both ways (rows to a multiple of 64, tokens to ldg, the
// token count rounded up to 64).  Then, on the same pipeline:
//  * grad_hidden += G . W_chunk, both operands stored [K][columns] (G by
//    vocabulary row, W_chunk as the lm_head rows are): transposing LDS reads
//    on both sides, the sum added into the fp32 output;
//  * grad_weight_chunk = G^T . hidden, K = tokens: G's rows are K-contiguous
//    and the hidden states are stored [K][columns], read in place with
//    transposing LDS reads (their rows past n_tokens are read as the last
//    one; G is zero there).
// All of it is queued on the caller's stream and works in the caller's
// workspace (bi_lmhead_backward) or in this file's static device array
// (bi_lmhead_backward_noalloc); nothing here allocates or synchronizes.  Every
// output element belongs to one workgroup of one launch, and the chunks
// follow each other on the stream, so grad_hidden's sum over chunks has a
// fixed order (no atomics): the result is the same bits on every run.

#include <hip/hip_runtime.h>

#include <mutex>

#include "bi_common.h"

// The device memory of bi_lmhead_backward_noalloc, for callers that cannot
// allocate: one chunk of G at a time.  Each GPU the library runs on holds its
// own copy of this array until the process ends.  In host code its name is
// only a stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device (see static_scratch).
static __device__ __align__(256) unsigned char scratch[BI_LMHEAD_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace bi_internal;

constexpr int64_t kChunkAlign = 256;   // lm_head rows per statistics tile
constexpr int64_t kKStage = 64;        // K per stage of the matrix-core pipeline
// tokens whose padded count (the products' K and G's row pitch) stays within
// the pipeline's 2^22-element row limit
constexpr int64_t kMaxTokens = (int64_t(1) << 22);

// token stride of the grad-logits chunk: a whole number of K stages
int64_t grad_ld(int64_t n_tokens) { return (n_tokens + kKStage - 1) / kKStage * kKStage; }

static_assert(int64_t(BI_LMHEAD_NOALLOC_MAX_TOKENS) * kChunkAlign * 2 ==
                  BI_LMHEAD_NOALLOC_SCRATCH_BYTES,
              "the static scratch holds one 256-row chunk of G at the most tokens");

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (the first call on a device) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];

int static_scratch(const char* fn, void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(BI_ERR_LAUNCH, "%s: no current HIP device (%s)", fn, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (r != hipSuccess || !ptr)
      return fail(BI_ERR_LAUNCH, "%s: hipGetSymbolAddress of the static scratch failed (%s)", fn,
                  hipGetErrorString(r));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return BI_OK;
}

// Host checks shared by both entry points; *empty when there is nothing to do.
int check_args(const char* fn, int64_t n_tokens, int64_t n_vocab_rows, int64_t d,
               int64_t hidden_stride, int64_t weight_stride, const float* lse,
               const float* grad_hidden, int64_t grad_hidden_stride, const void* grad_weight,
               int grad_weight_dtype, int64_t grad_weight_stride, bool* empty) {
  *empty = false;
  if (grad_weight_dtype != BI_F32 && grad_weight_dtype != BI_BF16)
    return fail(BI_ERR_DTYPE, "%s: grad_weight dtype %d", fn, grad_weight_dtype);
  if (n_tokens < 0 || n_vocab_rows < 0 || d < 1)
    return fail(BI_ERR_SHAPE, "%s: negative size", fn);
  const int64_t i32 = 0x7fffffff;
  if (n_vocab_rows > i32 || d > i32 || hidden_stride > i32 || weight_stride > i32 ||
      grad_hidden_stride > i32 || grad_weight_stride > i32)
    return fail(BI_ERR_SHAPE, "%s: sizes and strides must fit 32 bits", fn);
  if (n_tokens > kMaxTokens)
    return fail(BI_ERR_SHAPE, "%s: n_tokens %lld above %lld", fn, (long long)n_tokens,
                (long long)kMaxTokens);
  if (grad_hidden_stride < d || grad_weight_stride < d)
    return fail(BI_ERR_SHAPE, "%s: gradient strides must be >= d", fn);
  if (n_tokens == 0 || n_vocab_rows == 0) {
    *empty = true;
    return BI_OK;
  }
  if (!grad_hidden || !grad_weight || !lse)
    return fail(BI_ERR_NULL, "%s: lse, grad_hidden and grad_weight are required", fn);
  if (!aligned(grad_hidden, 4) || !aligned(grad_weight, grad_weight_dtype == BI_BF16 ? 2 : 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned gradient", fn);
  return BI_OK;
}

// The chunk loop, with G in `g` (256-byte aligned, ws_bytes long).
int run_chunks(const char* fn, const void* hidden, const void* weight, int64_t n_tokens,
               int64_t n_vocab_rows, int64_t d, int64_t hidden_stride, int64_t weight_stride,
               int64_t vocab_offset, int64_t vocab, const int64_t* labels, int64_t ignore_index,
               const float* lse, const float* token_weights, float* grad_hidden,
               int64_t grad_hidden_stride, void* grad_weight, int grad_weight_dtype,
               int64_t grad_weight_stride, uint16_t* g, int64_t ws_bytes, int32_t* status_flag,
               bi_stream_t stream) {
  const int64_t ldg = grad_ld(n_tokens);
  const int64_t fit = ws_bytes / (ldg * 2) / kChunkAlign * kChunkAlign;
  const int64_t chunk = fit < n_vocab_rows ? fit : n_vocab_rows;
  if (chunk < 1)
    return fail(BI_ERR_SHAPE, "%s: workspace of %lld bytes is below %lld", fn,
                (long long)ws_bytes, (long long)(kChunkAlign * ldg * 2));
  const size_t gw_elem = grad_weight_dtype == BI_BF16 ? 2 : 4;
  for (int64_t c0 = 0; c0 < n_vocab_rows; c0 += chunk) {
    const int64_t rows = n_vocab_rows - c0 < chunk ? n_vocab_rows - c0 : chunk;
    // G's rows up to the next multiple of 64 (within the chunk buffer, whose
    // row count is a multiple of 256 or covers the whole shard's last tile)
    const int64_t kpad = (rows + kKStage - 1) / kKStage * kKStage;
    const uint16_t* wc = static_cast<const uint16_t*>(weight) + c0 * weight_stride;
    if (int r = lmhead_grad_logits_padded(fn, hidden, wc, n_tokens, rows, d, hidden_stride,
                                          weight_stride, vocab_offset + c0, vocab, labels,
                                          ignore_index, lse, token_weights, g, ldg, kpad, ldg,
                                          status_flag, stream))
      return r;
    // grad_hidden[n][c] += sum_v G[v][n] W_c[v][c]; G's padding rows are zero
    if (int r = lmhead_product_t(fn, g, n_tokens, ldg, wc, d, weight_stride, kpad, rows,
                                 grad_hidden, grad_hidden_stride, stream))
      return r;
    // grad_weight_c[v][c] = sum_n G[v][n] hidden[n][c]; G's padding columns are zero
    void* gwc = static_cast<char*>(grad_weight) + c0 * grad_weight_stride * int64_t(gw_elem);
    if (int r = lmhead_product_nt(fn, g, rows, ldg, hidden, d, hidden_stride, ldg, n_tokens, gwc,
                                  grad_weight_stride, grad_weight_dtype == BI_BF16, stream))
      return r;
  }
  return launched(fn);
}

}  // namespace

extern "C" {

int64_t bi_lmhead_backward_workspace(int64_t n_tokens, int64_t d, int64_t chunk_rows) {
  if (n_tokens < 0 || d < 0 || chunk_rows < 1 || n_tokens > kMaxTokens) return -1;
  const int64_t rows = (chunk_rows + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  return rows * grad_ld(n_tokens) * 2;
}

int bi_lmhead_backward(const void* hidden, const void* weight, int64_t n_tokens,
                       int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                       int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                       const int64_t* labels, int64_t ignore_index, const float* lse,
                       const float* token_weights, float* grad_hidden,
                       int64_t grad_hidden_stride, void* grad_weight, int grad_weight_dtype,
                       int64_t grad_weight_stride, void* workspace, int64_t workspace_bytes,
                       int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_lmhead_backward";
  bool empty = false;
  if (int r = check_args(fn, n_tokens, n_vocab_rows, d, hidden_stride, weight_stride, lse,
                         grad_hidden, grad_hidden_stride, grad_weight, grad_weight_dtype,
                         grad_weight_stride, &empty))
    return r;
  if (empty) return ok();
  if (!workspace) return fail(BI_ERR_NULL, "%s: workspace is required", fn);
  if (!aligned(workspace, 256)) return fail(BI_ERR_ALIGN, "%s: workspace needs 256 bytes", fn);
  return run_chunks(fn, hidden, weight, n_tokens, n_vocab_rows, d, hidden_stride, weight_stride,
                    vocab_offset, vocab, labels, ignore_index, lse, token_weights, grad_hidden,
                    grad_hidden_stride, grad_weight, grad_weight_dtype, grad_weight_stride,
                    static_cast<uint16_t*>(workspace), workspace_bytes, status_flag, stream);
}

int bi_lmhead_backward_noalloc(const void* hidden, const void* weight, int64_t n_tokens,
                               int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                               int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                               const int64_t* labels, int64_t ignore_index, const float* lse,
                               const float* token_weights, float* grad_hidden,
                               int64_t grad_hidden_stride, void* grad_weight,
                               int grad_weight_dtype, int64_t grad_weight_stride,
                               int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_lmhead_backward_noalloc";
  bool empty = false;
  if (int r = check_args(fn, n_tokens, n_vocab_rows, d, hidden_stride, weight_stride, lse,
                         grad_hidden, grad_hidden_stride, grad_weight, grad_weight_dtype,
                         grad_weight_stride, &empty))
    return r;
  if (empty) return ok();
  if (n_tokens > BI_LMHEAD_NOALLOC_MAX_TOKENS)
    return fail(BI_ERR_SHAPE,
                "%s: n_tokens %lld above %d, the most for which one 256-row chunk of the "
                "logits gradient fits the %d-byte static scratch",
                fn, (long long)n_tokens, BI_LMHEAD_NOALLOC_MAX_TOKENS,
                BI_LMHEAD_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if (int r = static_scratch(fn, &ptr)) return r;
  return run_chunks(fn, hidden, weight, n_tokens, n_vocab_rows, d, hidden_stride, weight_stride,
                    vocab_offset, vocab, labels, ignore_index, lse, token_weights, grad_hidden,
                    grad_hidden_stride, grad_weight, grad_weight_dtype, grad_weight_stride,
                    static_cast<uint16_t*>(ptr), BI_LMHEAD_NOALLOC_SCRATCH_BYTES, status_flag,
                    stream);
}

}  // extern "C"
