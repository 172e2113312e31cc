// bi_lmhead_bwd.hip - the lm_head backward: gradients of the hidden states and
// of the lm_head rows from the saved lse, without the [N, V] logits or their
// gradient ever existing in full.  C ABI: bi_lmhead_backward,
// bi_lmhead_backward_workspace (include/bi_logprob.h).
//
// What is computed: with G[n, v] = w_n * (softmax(z_n)[v] - [v == y_n]) the
// cross-entropy backward of "[RL] Avoid full-vocab gather for TP policy
// statistics" (torchtitan PR #4685, Summary) on the lm_head logits
// z = hidden @ weight^T, the chain rule gives grad_hidden = G @ weight and
// grad_weight = G^T @ hidden: the chunked lm_head backward of
// "ZeroSyncGRPOTrainer" (bf16 GEMMs with fp32 accumulation).
//
// How: the vocabulary shard is cut into chunks of rows that fit the caller's
// workspace.  For each chunk, bi_lmhead_grad_logits recomputes its logits on
// the matrix cores (the forward's exact MFMA sequence) and writes G for the
// chunk as bf16, vocabulary-major [rows][n_tokens]; then two plain library
// GEMMs (rocBLAS, bf16 operands, fp32 accumulation) add G @ W_chunk into
// grad_hidden and write G^T @ hidden into the chunk's grad_weight rows.  All
// of it is queued on the caller's stream; rocBLAS works in the first part of
// the caller's workspace, so nothing here allocates device memory except the
// per-device rocBLAS handle, created on the first call on a device.

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "bi_common.h"

namespace {

using namespace bi_internal;

constexpr int64_t kBlasWorkspace = int64_t(32) << 20;   // rocBLAS's part of the workspace
constexpr int64_t kChunkAlign = 256;                    // lm_head rows per statistics tile
constexpr int kMaxDevices = 64;

// token stride of the grad-logits chunk: rows start on 16-byte boundaries
int64_t grad_ld(int64_t n_tokens) { return (n_tokens + 7) / 8 * 8; }

std::mutex g_blas_mutex;
rocblas_handle g_blas[kMaxDevices];

int blas_status(const char* fn, const char* what, rocblas_status st) {
  if (st == rocblas_status_success) return BI_OK;
  return fail(BI_ERR_LAUNCH, "%s: %s: %s", fn, what, rocblas_status_to_string(st));
}

// The calling thread's current device's handle (caller holds g_blas_mutex).
int blas_handle(const char* fn, rocblas_handle* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(BI_ERR_LAUNCH, "%s: no current HIP device", fn);
  if (!g_blas[dev]) {
    rocblas_handle h = nullptr;
    if (int r = blas_status(fn, "rocblas_create_handle", rocblas_create_handle(&h))) return r;
    // deterministic GEMMs: no atomics-based reductions
    if (int r = blas_status(fn, "rocblas_set_atomics_mode",
                            rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed)))
      return r;
    g_blas[dev] = h;
  }
  *out = g_blas[dev];
  return BI_OK;
}

}  // namespace

extern "C" {

int64_t bi_lmhead_backward_workspace(int64_t n_tokens, int64_t chunk_rows) {
  if (n_tokens < 0 || chunk_rows < 1) return -1;
  const int64_t rows = (chunk_rows + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  return kBlasWorkspace + rows * grad_ld(n_tokens) * 2;
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
  if (grad_weight_dtype != BI_F32 && grad_weight_dtype != BI_BF16)
    return fail(BI_ERR_DTYPE, "%s: grad_weight dtype %d", fn, grad_weight_dtype);
  if (n_tokens < 0 || n_vocab_rows < 0 || d < 1)
    return fail(BI_ERR_SHAPE, "%s: negative size", fn);
  const int64_t i32 = 0x7fffffff;
  if (n_tokens > i32 || n_vocab_rows > i32 || d > i32 || hidden_stride > i32 ||
      weight_stride > i32 || grad_hidden_stride > i32 || grad_weight_stride > i32 ||
      grad_ld(n_tokens) > i32)
    return fail(BI_ERR_SHAPE, "%s: sizes and strides must fit 32 bits", fn);
  if (grad_hidden_stride < d || grad_weight_stride < d)
    return fail(BI_ERR_SHAPE, "%s: gradient strides must be >= d", fn);
  if (n_tokens == 0 || n_vocab_rows == 0) return ok();
  if (!grad_hidden || !grad_weight || !workspace || !lse)
    return fail(BI_ERR_NULL, "%s: lse, grad_hidden, grad_weight and workspace are required", fn);
  if (!aligned(grad_hidden, 4) || !aligned(grad_weight, grad_weight_dtype == BI_BF16 ? 2 : 4) ||
      !aligned(workspace, 256))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer (workspace needs 256 bytes)", fn);
  const int64_t ldg = grad_ld(n_tokens);
  const int64_t fit = workspace_bytes > kBlasWorkspace
                          ? (workspace_bytes - kBlasWorkspace) / (ldg * 2) / kChunkAlign * kChunkAlign
                          : 0;
  const int64_t chunk = fit < n_vocab_rows ? fit : n_vocab_rows;
  if (chunk < 1)
    return fail(BI_ERR_SHAPE, "%s: workspace of %lld bytes is below %lld", fn,
                (long long)workspace_bytes,
                (long long)bi_lmhead_backward_workspace(n_tokens, kChunkAlign));
  uint16_t* g = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kBlasWorkspace);
  const size_t gw_elem = grad_weight_dtype == BI_BF16 ? 2 : 4;
  const rocblas_datatype gw_type =
      grad_weight_dtype == BI_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;

  std::lock_guard<std::mutex> lock(g_blas_mutex);
  rocblas_handle h = nullptr;
  if (int r = blas_handle(fn, &h)) return r;
  if (int r = blas_status(fn, "rocblas_set_stream",
                          rocblas_set_stream(h, static_cast<hipStream_t>(stream))))
    return r;
  if (int r = blas_status(fn, "rocblas_set_workspace",
                          rocblas_set_workspace(h, workspace, size_t(kBlasWorkspace))))
    return r;
  const float one = 1.0f, zero = 0.0f;
  for (int64_t c0 = 0; c0 < n_vocab_rows; c0 += chunk) {
    const int64_t rows = n_vocab_rows - c0 < chunk ? n_vocab_rows - c0 : chunk;
    const uint16_t* wc = static_cast<const uint16_t*>(weight) + c0 * weight_stride;
    if (int r = bi_lmhead_grad_logits(hidden, wc, n_tokens, rows, d, hidden_stride,
                                      weight_stride, vocab_offset + c0, vocab, labels,
                                      ignore_index, lse, token_weights, g, ldg, status_flag,
                                      stream))
      return r;
    // column-major view: grad_hidden^T (d x N) += W_c^T (d x rows) . (G^T: rows x N)
    if (int r = blas_status(
            fn, "rocblas_gemm_ex (grad_hidden)",
            rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_transpose, int(d),
                            int(n_tokens), int(rows), &one, wc, rocblas_datatype_bf16_r,
                            int(weight_stride), g, rocblas_datatype_bf16_r, int(ldg), &one,
                            grad_hidden, rocblas_datatype_f32_r, int(grad_hidden_stride),
                            grad_hidden, rocblas_datatype_f32_r, int(grad_hidden_stride),
                            rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0)))
      return r;
    // grad_weight_c^T (d x rows) = hidden^T (d x N) . G (N x rows)
    void* gwc = static_cast<char*>(grad_weight) + c0 * grad_weight_stride * int64_t(gw_elem);
    if (int r = blas_status(
            fn, "rocblas_gemm_ex (grad_weight)",
            rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, int(d), int(rows),
                            int(n_tokens), &one, hidden, rocblas_datatype_bf16_r,
                            int(hidden_stride), g, rocblas_datatype_bf16_r, int(ldg), &zero, gwc,
                            gw_type, int(grad_weight_stride), gwc, gw_type,
                            int(grad_weight_stride), rocblas_datatype_f32_r,
                            rocblas_gemm_algo_standard, 0, 0)))
      return r;
  }
  return launched(fn);
}

}  // extern "C"
