// bi_common.h - device helpers shared by the HIP translation units of
// libbi_logprob (bi_logprob.hip: row kernels; bi_lmhead.hip: lm_head GEMM with
// statistics), and the library's error state.  Internal: not installed, not
// part of the C ABI.
//
// The lane accumulator keeps, in the log2 domain about a reference c (a
// rounded -m*log2e for the running max m), S = sum 2^t and U = sum 2^t * t with
// t = fma(z, log2e, c): the softmax denominator and the entropy-weighted sum
// of "[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan PR
// #4685), Summary and Why, in a form that needs one FMA and one exp2 per logit.
#pragma once

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bi_logprob.h"

namespace bi_internal {

// Error text of the calling thread's last failed call (bi_last_error).
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();
bool aligned(const void* p, size_t a);
int launched(const char* what);
const char* last_error();

// D[i][j] = sum_k A[i][k] B[k][j] on the lm_head kernel's matrix-core
// pipeline: A [m][k] bf16 with rows of k contiguous elements (zero in its
// columns kvalid_b .. k-1), B [k][n] bf16 with rows of n contiguous elements,
// of which rows kvalid_b .. k-1 (fewer than 64) are read as its last one; k a
// multiple of 64; D fp32 or bf16, overwritten.  Used by the lm_head backward.
int lmhead_product_nt(const char* fn, const void* a, int64_t m, int64_t lda, const void* b,
                      int64_t n, int64_t ldb, int64_t k, int64_t kvalid_b, void* d, int64_t ldd,
                      bool d_bf16, bi_stream_t stream);

// D[i][j] += sum_k A[k][i] B[k][j] on the same pipeline with transposing LDS
// reads: A [k][m] and B [k][n] bf16 with rows of m (n) contiguous elements; k
// a multiple of 64; B's rows from kvalid_b on (fewer than 64) are read as its
// last one, so A must be zero there; D fp32, added into.
int lmhead_product_t(const char* fn, const void* a, int64_t m, int64_t lda, const void* b,
                     int64_t n, int64_t ldb, int64_t k, int64_t kvalid_b, float* d, int64_t ldd,
                     bi_stream_t stream);

// bi_lmhead_grad_logits that also writes rows n_vocab_rows .. pad_rows - 1
// and columns n_tokens .. pad_cols - 1 of the gradient as zeros (pad_rows
// within the last 256-row tile, pad_cols within the last 256-token tile).
int lmhead_grad_logits_padded(const char* fn, const void* hidden, const void* weight,
                              int64_t n_tokens, int64_t n_vocab_rows, int64_t d,
                              int64_t hidden_stride, int64_t weight_stride, int64_t vocab_offset,
                              int64_t vocab, const int64_t* labels, int64_t ignore_index,
                              const float* lse, const float* token_weights, void* grad_logits,
                              int64_t grad_stride, int64_t pad_rows, int64_t pad_cols,
                              int32_t* status_flag, bi_stream_t stream);

}  // namespace bi_internal

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kTFloor = -256.0f;   // 2^t == 0 in fp32 for every t below this

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_max3_f32 without the canonicalizing moves fmaxf would add around
// non-arithmetic inputs (decoded bits).  NaN inputs still reach the sums.
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// log2-domain reference of a running max: c = -RN(m*log2e), kept finite for
// m = -inf (an empty lane) so that no inf - inf arises.
__device__ inline float ref_of(float m) { return fminf(-(m * kLog2e), FLT_MAX); }

// --------------------------------------------------------- lane accumulator

struct Acc {
  float m;  // running max of the logits seen
  float c;  // ref_of(m)
  float S;  // sum of 2^t
  float U;  // sum of 2^t * t   (log2 units, about c)
};

__device__ inline Acc acc_empty() { return Acc{-INFINITY, FLT_MAX, 0.0f, 0.0f}; }

// Move an accumulator to the reference C (C <= a.c).  Exact no-op for C == a.c.
__device__ inline void rebase(Acc& a, float C) {
  const float d = fmaxf(C - a.c, kTFloor);
  const float f = exp2_hw(d);
  a.U = f * fmaf(d, a.S, a.U);
  a.S = f * a.S;
  a.c = C;
}

// max of K values through a fixed tree of v_max3 (K - 1 values removed per
// two-operand step, so ceil((K - 1) / 2) instructions)
template <int K>
__device__ inline float max_reduce(const float* v) {
  if constexpr (K == 1) {
    return v[0];
  } else if constexpr (K == 2) {
    return max3(v[0], v[1], v[1]);
  } else {
    constexpr int Q = K / 3, R = K % 3;
    float w[Q + R];
#pragma unroll
    for (int j = 0; j < Q; ++j) w[j] = max3(v[3 * j], v[3 * j + 1], v[3 * j + 2]);
#pragma unroll
    for (int r = 0; r < R; ++r) w[Q + r] = v[3 * Q + r];
    return max_reduce<Q + R>(w);
  }
}

template <int N>
__device__ inline float tree_max(const float* z, float m) {
  float v[N + 1];
  v[0] = m;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i + 1] = z[i];
  return max_reduce<N + 1>(v);
}

template <int VEC>
__device__ inline float tree_sum(const float* e) {
  if constexpr (VEC == 8) {
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  } else {
    return (e[0] + e[1]) + (e[2] + e[3]);
  }
}

// The two halves of accumulate.  First the group's max over its N values
// moves `a` to the new reference, which is returned ...
template <int N>
__device__ inline float accumulate_rebase(Acc& a, const float* z) {
  const float mx = tree_max<N>(z, a.m);
  const float c = ref_of(mx);
  rebase(a, c);
  a.m = mx;
  return c;
}

// ... then each vector's VEC values add their terms about it.
template <int VEC>
__device__ inline void accumulate_terms(Acc& a, const float* z, float c) {
  float e[VEC], tc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const float t = fmaf(z[k], kLog2e, c);
    e[k] = exp2_hw(t);              // 0 for z = -inf; NaN for NaN z
    tc[k] = fmaxf(t, kTFloor);      // finite, so 0 * tc == 0 for masked columns
  }
  float u = e[0] * tc[0];
#pragma unroll
  for (int k = 1; k < VEC; ++k) u = fmaf(e[k], tc[k], u);
  a.S += tree_sum<VEC>(e);
  a.U += u;
}

// Accumulate NV vectors (NV*VEC decoded values, in lane order) into `a`.
template <int VEC, int NV>
__device__ inline void accumulate(Acc& a, const float* z) {
  const float c = accumulate_rebase<NV * VEC>(a, z);
#pragma unroll
  for (int j = 0; j < NV; ++j) accumulate_terms<VEC>(a, z + j * VEC, c);
}

}  // namespace
