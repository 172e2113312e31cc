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
// workspace.  For each chunk, the grad-logits kernel recomputes its logits on
// the matrix cores (the forward's exact MFMA sequence) and writes G for the
// chunk as bf16, vocabulary-major [rows][n_tokens], its rows padded with
// zeros to a multiple of 64; then G @ W_chunk is added into grad_hidden and
// G^T @ hidden written into the chunk's grad_weight rows (bf16 operands, fp32
// accumulation).  G @ W_chunk has both operands stored [K][columns] (G by
// vocabulary row, W_chunk as the lm_head rows are): it runs on the lm_head
// kernel's pipeline with transposing LDS reads.  G^T @ hidden has G's rows,
// token-contiguous, as one operand: when n_tokens is a multiple of 64 (at
// most 2^22) and the workspace holds a transposed copy of the hidden states
// ([d][n_tokens], made once per call), it runs on the same pipeline.  Outside
// those limits a product runs on hipBLASLt (a plain library GEMM), which
// works in the first part of the caller's workspace.  All of it is queued on
// the caller's stream; nothing here allocates device memory except the
// per-device hipBLASLt handle, created on the first call that needs it.  The
// algorithm of each library GEMM shape is chosen once by hipBLASLt's
// heuristic and kept, so a shape always runs the same kernel.

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

// G^T @ hidden on the matrix-core pipeline needs the token count to be a
// whole number of its 64-wide K stages (and within its 2^22 limit)
bool own_product(int64_t n_tokens) {
  return n_tokens % 64 == 0 && n_tokens <= (int64_t(1) << 22);
}

// bytes of the transposed hidden states [d][n_tokens] in the workspace
int64_t transposed_bytes(int64_t n_tokens, int64_t d) {
  return own_product(n_tokens) ? (d * n_tokens * 2 + 255) / 256 * 256 : 0;
}

// ht[c][n] = h[n][c] for a 64 x 64 block per workgroup (n_tokens and d are
// multiples of 64, rows 16-byte aligned): 16-byte loads, a padded LDS tile,
// 16-byte stores.
constexpr int kTp = 64;
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ h,
                                                         int64_t ldh, uint16_t* __restrict__ ht,
                                                         int64_t ldht) {
  __shared__ uint16_t tile[kTp][kTp + 8];
  const int64_t n0 = int64_t(blockIdx.x) * kTp, c0 = int64_t(blockIdx.y) * kTp;
  for (int q = threadIdx.x; q < kTp * kTp / 8; q += 256) {
    const int n = q / (kTp / 8), cc = 8 * (q % (kTp / 8));
    const u32x4 v = *reinterpret_cast<const u32x4*>(h + (n0 + n) * ldh + c0 + cc);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[cc + e][n] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTp * kTp / 8; q += 256) {
    const int c = q / (kTp / 8), nn = 8 * (q % (kTp / 8));
    u32x4 v;
    v.x = uint32_t(tile[c][nn + 0]) | (uint32_t(tile[c][nn + 1]) << 16);
    v.y = uint32_t(tile[c][nn + 2]) | (uint32_t(tile[c][nn + 3]) << 16);
    v.z = uint32_t(tile[c][nn + 4]) | (uint32_t(tile[c][nn + 5]) << 16);
    v.w = uint32_t(tile[c][nn + 6]) | (uint32_t(tile[c][nn + 7]) << 16);
    *reinterpret_cast<u32x4*>(ht + (c0 + c) * ldht + n0 + nn) = v;
  }
}

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

int64_t bi_lmhead_backward_workspace(int64_t n_tokens, int64_t d, int64_t chunk_rows) {
  if (n_tokens < 0 || d < 0 || chunk_rows < 1) return -1;
  const int64_t rows = (chunk_rows + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  return kBlasWorkspace + transposed_bytes(n_tokens, d) + rows * grad_ld(n_tokens) * 2;
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
  // the transposed hidden states when G^T @ hidden can run on the matrix-core
  // pipeline and the workspace holds them beside one chunk; else the library
  int64_t ht_bytes = transposed_bytes(n_tokens, d);
  if (workspace_bytes < kBlasWorkspace + ht_bytes + kChunkAlign * ldg * 2) ht_bytes = 0;
  const bool own = ht_bytes > 0;
  const int64_t room = workspace_bytes - kBlasWorkspace - ht_bytes;
  const int64_t fit = room > 0 ? room / (ldg * 2) / kChunkAlign * kChunkAlign : 0;
  const int64_t chunk = fit < n_vocab_rows ? fit : n_vocab_rows;
  if (chunk < 1)
    return fail(BI_ERR_SHAPE, "%s: workspace of %lld bytes is below %lld", fn,
                (long long)workspace_bytes,
                (long long)(bi_lmhead_backward_workspace(n_tokens, d, kChunkAlign) -
                            transposed_bytes(n_tokens, d)));
  char* ws = static_cast<char*>(workspace);
  uint16_t* ht = reinterpret_cast<uint16_t*>(ws + kBlasWorkspace);
  uint16_t* g = reinterpret_cast<uint16_t*>(ws + kBlasWorkspace + ht_bytes);
  const size_t gw_elem = grad_weight_dtype == BI_BF16 ? 2 : 4;
  // grad_hidden += G . W_c on the matrix-core pipeline with transposing reads
  // (G vocabulary-major and W_c as stored are both [K][columns]) while G's
  // row pitch is within its limit; else on the library
  const bool own_dh = ldg <= (int64_t(1) << 22);

  std::unique_lock<std::mutex> lock(g_blas_mutex, std::defer_lock);
  int dev = -1;
  hipblasLtHandle_t h = nullptr;
  if (!own || !own_dh) {   // the library is needed: its handle, made once per device
    lock.lock();
    if (int r = lt_handle(fn, &dev, &h)) return r;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipDataType gw_type = grad_weight_dtype == BI_BF16 ? HIP_R_16BF : HIP_R_32F;
  if (own) {
    if (d % kTp != 0 || !aligned(hidden, 16) || hidden_stride % 8 != 0)
      return fail(BI_ERR_SHAPE, "%s: d must be a multiple of 64 with 16-byte hidden rows", fn);
    hipLaunchKernelGGL(transpose_kernel, dim3(unsigned(n_tokens / kTp), unsigned(d / kTp)),
                       dim3(256), 0, s, static_cast<const uint16_t*>(hidden), hidden_stride, ht,
                       n_tokens);
    if (int r = launched(fn)) return r;
  }
  for (int64_t c0 = 0; c0 < n_vocab_rows; c0 += chunk) {
    const int64_t rows = n_vocab_rows - c0 < chunk ? n_vocab_rows - c0 : chunk;
    // G's rows up to the next multiple of 64 (within the chunk buffer, whose
    // row count is a multiple of 256 or covers the whole shard's last tile)
    const int64_t kpad = (rows + 63) / 64 * 64;
    const uint16_t* wc = static_cast<const uint16_t*>(weight) + c0 * weight_stride;
    if (int r = lmhead_grad_logits_padded(fn, hidden, wc, n_tokens, rows, d, hidden_stride,
                                          weight_stride, vocab_offset + c0, vocab, labels,
                                          ignore_index, lse, token_weights, g, ldg,
                                          own_dh ? kpad : rows, status_flag, stream))
      return r;
    if (own_dh) {
      // grad_hidden[n][c] += sum_v G[v][n] W_c[v][c]; G's padding rows are zero
      if (int r = lmhead_product_t(fn, g, n_tokens, ldg, wc, d, weight_stride, kpad, rows,
                                   grad_hidden, grad_hidden_stride, stream))
        return r;
    } else {
      // column-major view: grad_hidden^T (d x N) += W_c^T (d x rows) . (G^T: rows x N)
      const Gemm dh{HIPBLAS_OP_N, HIPBLAS_OP_T, d, n_tokens, rows, weight_stride, ldg,
                    grad_hidden_stride, HIP_R_32F};
      if (int r = lt_gemm(fn, h, dev, dh, wc, g, 1.0f, grad_hidden, workspace,
                          size_t(kBlasWorkspace), s))
        return r;
    }
    void* gwc = static_cast<char*>(grad_weight) + c0 * grad_weight_stride * int64_t(gw_elem);
    if (own) {
      // grad_weight_c[v][c] = sum_n G[v][n] ht[c][n]
      if (int r = lmhead_product(fn, g, rows, ldg, ht, d, n_tokens, n_tokens, gwc,
                                 grad_weight_stride, grad_weight_dtype == BI_BF16, stream))
        return r;
    } else {
      // grad_weight_c^T (d x rows) = hidden^T (d x N) . G (N x rows)
      const Gemm dw{HIPBLAS_OP_N, HIPBLAS_OP_N, d, rows, n_tokens, hidden_stride, ldg,
                    grad_weight_stride, gw_type};
      if (int r = lt_gemm(fn, h, dev, dw, hidden, g, 0.0f, gwc, workspace,
                          size_t(kBlasWorkspace), s))
        return r;
    }
  }
  return launched(fn);
}

}  // extern "C"
