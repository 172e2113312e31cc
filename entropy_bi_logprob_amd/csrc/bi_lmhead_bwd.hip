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
// GEMMs (hipBLASLt, bf16 operands, fp32 accumulation) add G @ W_chunk into
// grad_hidden and write G^T @ hidden into the chunk's grad_weight rows.  All
// of it is queued on the caller's stream; hipBLASLt works in the first part
// of the caller's workspace, so nothing here allocates device memory except
// the per-device hipBLASLt handle, created on the first call on a device.
// The algorithm of each GEMM shape is chosen once by hipBLASLt's heuristic
// and kept, so a shape always runs the same kernel (reproducible results).

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "bi_common.h"

namespace {

using namespace bi_internal;

constexpr int64_t kBlasWorkspace = int64_t(128) << 20;  // hipBLASLt's part of the workspace
constexpr int64_t kChunkAlign = 256;                    // lm_head rows per statistics tile
constexpr int kMaxDevices = 64;

// token stride of the grad-logits chunk: rows start on 16-byte boundaries
int64_t grad_ld(int64_t n_tokens) { return (n_tokens + 7) / 8 * 8; }

std::mutex g_blas_mutex;
hipblasLtHandle_t g_lt[kMaxDevices];

// column-major D = op(A) op(B) + beta C, bf16 A and B, fp32 accumulation
struct Gemm {
  hipblasOperation_t ta, tb;
  int64_t m, n, k, lda, ldb, ldc;
  hipDataType ct;   // type of C and D
  auto key(int dev) const {
    return std::make_tuple(dev, int(ta), int(tb), m, n, k, lda, ldb, ldc, int(ct));
  }
};

std::map<std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int>,
         hipblasLtMatmulAlgo_t>
    g_algos;

int lt_status(const char* fn, const char* what, hipblasStatus_t st) {
  if (st == HIPBLAS_STATUS_SUCCESS) return BI_OK;
  return fail(BI_ERR_LAUNCH, "%s: %s failed (hipblasStatus %d)", fn, what, int(st));
}

// The calling thread's current device and its handle (caller holds g_blas_mutex).
int lt_handle(const char* fn, int* dev_out, hipblasLtHandle_t* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(BI_ERR_LAUNCH, "%s: no current HIP device", fn);
  if (!g_lt[dev]) {
    hipblasLtHandle_t h = nullptr;
    if (int r = lt_status(fn, "hipblasLtCreate", hipblasLtCreate(&h))) return r;
    g_lt[dev] = h;
  }
  *dev_out = dev;
  *out = g_lt[dev];
  return BI_OK;
}

// Descriptors of one GEMM (host objects, released by the destructor).
struct GemmDesc {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  ~GemmDesc() {
    if (c) hipblasLtMatrixLayoutDestroy(c);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

int lt_gemm(const char* fn, hipblasLtHandle_t h, int dev, const Gemm& g, const void* A,
            const void* B, float beta, void* C, void* ws, size_t ws_bytes, hipStream_t s) {
  GemmDesc d;
  const int32_t ta = g.ta, tb = g.tb;
  if (int r = lt_status(fn, "matmul descriptor",
                        hipblasLtMatmulDescCreate(&d.op, HIPBLAS_COMPUTE_32F, HIP_R_32F)))
    return r;
  if (int r = lt_status(fn, "transposes",
                        hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta,
                                                        sizeof(ta))))
    return r;
  if (int r = lt_status(fn, "transposes",
                        hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb,
                                                        sizeof(tb))))
    return r;
  const bool na = g.ta == HIPBLAS_OP_N, nb = g.tb == HIPBLAS_OP_N;
  if (int r = lt_status(fn, "layouts",
                        hipblasLtMatrixLayoutCreate(&d.a, HIP_R_16BF, na ? g.m : g.k,
                                                    na ? g.k : g.m, g.lda)))
    return r;
  if (int r = lt_status(fn, "layouts",
                        hipblasLtMatrixLayoutCreate(&d.b, HIP_R_16BF, nb ? g.k : g.n,
                                                    nb ? g.n : g.k, g.ldb)))
    return r;
  if (int r = lt_status(fn, "layouts", hipblasLtMatrixLayoutCreate(&d.c, g.ct, g.m, g.n, g.ldc)))
    return r;
  auto it = g_algos.find(g.key(dev));
  if (it == g_algos.end()) {
    hipblasLtMatmulPreference_t pref = nullptr;
    if (int r = lt_status(fn, "preference", hipblasLtMatmulPreferenceCreate(&pref))) return r;
    const uint64_t max_ws = ws_bytes;
    constexpr int kAsk = 8;
    hipblasLtMatmulHeuristicResult_t res[kAsk];
    int found = 0;
    hipblasStatus_t st = hipblasLtMatmulPreferenceSetAttribute(
        pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws, sizeof(max_ws));
    if (st == HIPBLAS_STATUS_SUCCESS)
      st = hipblasLtMatmulAlgoGetHeuristic(h, d.op, d.a, d.b, d.c, d.c, pref, kAsk, res, &found);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (int r = lt_status(fn, "algorithm heuristic", st)) return r;
    int pick = -1;   // the heuristic's first choice that fits the workspace
    for (int i = 0; i < found && pick < 0; ++i)
      if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= ws_bytes) pick = i;
    if (pick < 0)
      return fail(BI_ERR_LAUNCH,
                  "%s: no GEMM algorithm for %lld x %lld x %lld within %zu workspace bytes "
                  "(%d candidates)", fn, (long long)g.m, (long long)g.n, (long long)g.k,
                  ws_bytes, found);
    it = g_algos.emplace(g.key(dev), res[pick].algo).first;
  }
  const float one = 1.0f;
  return lt_status(fn, "hipblasLtMatmul",
                   hipblasLtMatmul(h, d.op, &one, A, d.a, B, d.b, &beta, C, d.c, C, d.c,
                                   &it->second, ws, ws_bytes, s));
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

  std::lock_guard<std::mutex> lock(g_blas_mutex);
  int dev = -1;
  hipblasLtHandle_t h = nullptr;
  if (int r = lt_handle(fn, &dev, &h)) return r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipDataType gw_type = grad_weight_dtype == BI_BF16 ? HIP_R_16BF : HIP_R_32F;
  for (int64_t c0 = 0; c0 < n_vocab_rows; c0 += chunk) {
    const int64_t rows = n_vocab_rows - c0 < chunk ? n_vocab_rows - c0 : chunk;
    const uint16_t* wc = static_cast<const uint16_t*>(weight) + c0 * weight_stride;
    if (int r = bi_lmhead_grad_logits(hidden, wc, n_tokens, rows, d, hidden_stride,
                                      weight_stride, vocab_offset + c0, vocab, labels,
                                      ignore_index, lse, token_weights, g, ldg, status_flag,
                                      stream))
      return r;
    // column-major view: grad_hidden^T (d x N) += W_c^T (d x rows) . (G^T: rows x N)
    const Gemm dh{HIPBLAS_OP_N, HIPBLAS_OP_T, d, n_tokens, rows, weight_stride, ldg,
                  grad_hidden_stride, HIP_R_32F};
    if (int r = lt_gemm(fn, h, dev, dh, wc, g, 1.0f, grad_hidden, workspace,
                        size_t(kBlasWorkspace), s))
      return r;
    // grad_weight_c^T (d x rows) = hidden^T (d x N) . G (N x rows)
    void* gwc = static_cast<char*>(grad_weight) + c0 * grad_weight_stride * int64_t(gw_elem);
    const Gemm dw{HIPBLAS_OP_N, HIPBLAS_OP_N, d, rows, n_tokens, hidden_stride, ldg,
                  grad_weight_stride, gw_type};
    if (int r = lt_gemm(fn, h, dev, dw, hidden, g, 0.0f, gwc, workspace, size_t(kBlasWorkspace),
                        s))
      return r;
  }
  return launched(fn);
}

}  // extern "C"
