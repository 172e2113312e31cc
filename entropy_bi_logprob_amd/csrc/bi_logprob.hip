// bi_logprob.hip - HIP kernels for gfx950 (CDNA4) and the C ABI declared in
// include/bi_logprob.h: batch-invariant per-token logprob, entropy, gradient
// and vocabulary-chunk statistics over large-vocabulary logits.
//
// What is computed comes from "[RL] Avoid full-vocab gather for TP policy
// statistics" (torchtitan PR #4685): Summary and Why (logprob, exact entropy
// from the global maximum, softmax denominator, target contribution and
// entropy-weighted sum; gradient from the cross-entropy backward), Correctness
// and compatibility (ignored labels, masked logits, weights, FP32/BF16, uneven
// vocabulary), and the review reply "Batch invariance under the patched
// logprob path" (bit equality needs a fixed summation grouping; max combines
// exactly, sums do not).  How it is computed here is this file's own design.
//
// Design (all of it memory-bound; no matrix cores):
//  * One workgroup reduces one row.  Its size T, the 16-byte vector width VEC
//    and the rescale group are functions of (dtype, width) only.  Lane t owns
//    the vectors v = k*T + t (k = 0, 1, ...) of the row, column v*VEC + s in
//    slot s; vectors past the row's end are read as -inf, which adds exactly
//    nothing.  The lane -> wave -> workgroup reduction tree is fixed.  Hence
//    every row's bits are independent of the batch it sits in.
//  * Each lane keeps (m, c, S, U) with a log2-domain reference c = -RN(m*log2e):
//    S = sum 2^t, U = sum 2^t * t, t = fma(z, log2e, c).  One FMA and one
//    v_exp_f32 per element; the reference is updated once per group of 16
//    elements with an exact, always-executed rescale (a no-op when m is
//    unchanged).  At the end lse = m + ln2*(log2 S - d) with the exact
//    residual d = fma(m, log2e, c), and entropy = ln2*(log2 S - U/S).
//  * -inf columns give 2^t = 0 and a clamped t (the 0 * -inf of the entropy
//    term becomes 0); NaN logits still propagate through S.
//  * The backward is elementwise from the saved lse: p = 2^((z - lse)*log2e),
//    grad = w*p, and w*(p - 1) at the label column.
//  * Loads and stores are 128-bit and non-temporal.  Rows need only be
//    aligned to 4 bytes for vector access (gfx9 global loads accept
//    dword-aligned dwordx4); bf16 rows on a 2-byte boundary take an element
//    path with the same column map and arithmetic.


#include <atomic>

#include "bi_common.h"

namespace {

using namespace bi_internal;

constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / 64;
constexpr int64_t kMaxWidth = int64_t(1) << 29;

#ifndef BI_GROUP_ELEMS
#define BI_GROUP_ELEMS 16
#endif
#ifndef BI_MIN_VECS_PER_LANE
#define BI_MIN_VECS_PER_LANE 32
#endif
constexpr int kGroupElems = BI_GROUP_ELEMS;   // elements per lane per rescale

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

struct Geometry {
  int threads;  // workgroup size
  int vec;      // elements per 16-byte vector
  int group;    // vectors per rescale group
};

// The batch-invariance contract: a function of (dtype, width) only.
__host__ __device__ inline Geometry row_geometry(int dtype, int64_t width) {
  Geometry g;
  g.vec = dtype == BI_BF16 ? 8 : 4;
  g.group = kGroupElems / g.vec;
  const int64_t nvec = (width + g.vec - 1) / g.vec;
  int t = 64;
  while (t < kMaxThreads && int64_t(t) * BI_MIN_VECS_PER_LANE < nvec) t *= 2;
  g.threads = t;
  return g;
}

// ------------------------------------------------------------------ elements

template <int DT>
struct Elt;

template <>
struct Elt<BI_F32> {
  static constexpr int VEC = 4;
  __device__ static inline void decode(const u32x4& r, float* z) {
    z[0] = __uint_as_float(r.x);
    z[1] = __uint_as_float(r.y);
    z[2] = __uint_as_float(r.z);
    z[3] = __uint_as_float(r.w);
  }
  __device__ static inline float load1(const char* row, int64_t j) {
    return reinterpret_cast<const float*>(row)[j];
  }
};

template <>
struct Elt<BI_BF16> {
  static constexpr int VEC = 8;
  // element 2k is the low half of dword k (little endian)
  __device__ static inline void decode(const u32x4& r, float* z) {
    z[0] = __uint_as_float(r.x << 16);
    z[1] = __uint_as_float(r.x & 0xffff0000u);
    z[2] = __uint_as_float(r.y << 16);
    z[3] = __uint_as_float(r.y & 0xffff0000u);
    z[4] = __uint_as_float(r.z << 16);
    z[5] = __uint_as_float(r.z & 0xffff0000u);
    z[6] = __uint_as_float(r.w << 16);
    z[7] = __uint_as_float(r.w & 0xffff0000u);
  }
  __device__ static inline float load1(const char* row, int64_t j) {
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(row)[j]) << 16);
  }
};

// Where one lane reads its vectors of a row.  Vector k*T + tid of the row
// (step k) sits at byte k*T*16 + tid*16.  The 4-byte-aligned path reads it
// with one non-temporal buffer_load_dwordx4: the lane's offset is a constant
// VGPR and the step offset an SGPR, so addressing costs no vector ALU.  A bf16
// row on a 2-byte boundary is read with element loads into the same bits.
struct RowSrc {
  __amdgpu_buffer_rsrc_t rs;
  const char* row;
  uint32_t lane_off;    // tid * 16
  uint32_t step_bytes;  // T * 16
};

#ifndef BI_LOAD_POLICY
#define BI_LOAD_POLICY 2
#endif
#ifndef BI_STORE_NT
#define BI_STORE_NT 1
#endif
constexpr int kNonTemporal = BI_LOAD_POLICY;   // buffer-load cache policy bits (2 = nt)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

__device__ inline RowSrc row_src(const char* row, int64_t row_bytes, int T, int tid) {
  RowSrc s;
  s.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), (short)0,
                                           int(row_bytes), kRsrcWord3);
  s.row = row;
  s.lane_off = uint32_t(tid) * 16u;
  s.step_bytes = uint32_t(T) * 16u;
  return s;
}

template <bool VLOAD, int POL = kNonTemporal>
__device__ inline u32x4 fetch(const RowSrc& s, uint32_t k) {
  if constexpr (VLOAD) {
    return __builtin_amdgcn_raw_buffer_load_b128(s.rs, s.lane_off, k * s.step_bytes, POL);
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(s.row + k * s.step_bytes + s.lane_off);
    u32x4 r;
    r.x = uint32_t(p[0]) | (uint32_t(p[1]) << 16);
    r.y = uint32_t(p[2]) | (uint32_t(p[3]) << 16);
    r.z = uint32_t(p[4]) | (uint32_t(p[5]) << 16);
    r.w = uint32_t(p[6]) | (uint32_t(p[7]) << 16);
    return r;
  }
}


template <int DT, int G, bool VLOAD, int POL = kNonTemporal>
__device__ inline void load_group(u32x4* buf, const RowSrc& src, uint32_t g) {
#pragma unroll
  for (int i = 0; i < G; ++i) buf[i] = fetch<VLOAD, POL>(src, g * G + i);
}

// Run body(buffer, g) over groups g = 0 .. n-1 of G steps each, with group
// g+1's loads issued before group g is processed.  Two register buffers are
// used in turn and the last group is peeled, so that every processing site
// sees the same unconditional loads ahead of it and waits only for its own.
// REV visits the groups from last to first (the order does not matter to an
// elementwise body; it is used to re-read the most recently loaded data first).
template <int DT, int G, bool VLOAD, int POL = kNonTemporal, bool REV = false, typename Body>
__device__ inline void pipelined_groups(const RowSrc& src, uint32_t n, Body&& body) {
  if (n == 0) return;
  auto at = [n](uint32_t g) { return REV ? n - 1 - g : g; };
  u32x4 A[G], B[G];
  load_group<DT, G, VLOAD, POL>(A, src, at(0));
  for (uint32_t g = 0;;) {
    if (g + 1 == n) {
      body(A, at(g));
      return;
    }
    load_group<DT, G, VLOAD, POL>(B, src, at(g + 1));
    body(A, at(g));
    ++g;
    if (g + 1 == n) {
      body(B, at(g));
      return;
    }
    load_group<DT, G, VLOAD, POL>(A, src, at(g + 1));
    body(B, at(g));
    ++g;
  }
}

template <int DT, int G>
__device__ inline void accumulate_group(Acc& a, const u32x4* buf) {
  constexpr int VEC = Elt<DT>::VEC;
  float z[G * VEC];
#pragma unroll
  for (int i = 0; i < G; ++i) Elt<DT>::decode(buf[i], z + i * VEC);
  accumulate<VEC, G>(a, z);
}

// Scan one row segment of `width` columns: every lane accumulates its vectors.
// Full groups run with the next group's loads in flight (two register
// buffers used in turn), then single full steps, then the one ragged step.
template <int DT, bool VLOAD, int POL = kNonTemporal>
__device__ inline void row_scan(Acc& a, const RowSrc& src, int64_t width, int T, int tid) {
  constexpr int VEC = Elt<DT>::VEC;
  constexpr int G = kGroupElems / VEC;
  const uint32_t nfull = uint32_t(width / VEC);
  const uint32_t nvec = uint32_t((width + VEC - 1) / VEC);
  const uint32_t full_steps = nfull / uint32_t(T);
  const uint32_t ngroups = full_steps / G;

  pipelined_groups<DT, G, VLOAD, POL>(src, ngroups, [&](const u32x4* buf, uint32_t) {
    accumulate_group<DT, G>(a, buf);
  });
  for (uint32_t k = ngroups * G; k < full_steps; ++k) {
    float z[VEC];
    Elt<DT>::decode(fetch<VLOAD, POL>(src, k), z);
    accumulate<VEC, 1>(a, z);
  }
  if (full_steps * uint32_t(T) < nvec) {
    const uint32_t v = full_steps * uint32_t(T) + tid;
    float z[VEC];
    if (v < nfull) {
      Elt<DT>::decode(fetch<VLOAD, POL>(src, full_steps), z);
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const int64_t j = int64_t(v) * VEC + k;
        z[k] = j < width ? Elt<DT>::load1(src.row, j) : -INFINITY;
      }
    }
    accumulate<VEC, 1>(a, z);
  }
}

// ------------------------------------------------- fixed reduction tree

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ inline float swizzle_xor16(float x) {
  // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ inline float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// max / sum over each 16-lane row (result in every lane of the row)
__device__ inline float row16_max(float m) {
  m = fmaxf(m, dpp<kQuadXor1>(m));
  m = fmaxf(m, dpp<kQuadXor2>(m));
  m = fmaxf(m, dpp<kRowHalfMirror>(m));
  return fmaxf(m, dpp<kRowMirror>(m));
}
__device__ inline float row16_sum(float s) {
  s = s + dpp<kQuadXor1>(s);
  s = s + dpp<kQuadXor2>(s);
  s = s + dpp<kRowHalfMirror>(s);
  return s + dpp<kRowMirror>(s);
}
// whole wave: rows -> halves (swizzle) -> lanes 0 and 32 (uniform result)
__device__ inline float wave_max(float m) {
  m = row16_max(m);
  m = fmaxf(m, swizzle_xor16(m));
  return fmaxf(lane_value(m, 0), lane_value(m, 32));
}
__device__ inline float wave_sum(float s) {
  s = row16_sum(s);
  s = s + swizzle_xor16(s);
  return lane_value(s, 0) + lane_value(s, 32);
}

// Reduce the lanes' accumulators of one workgroup; the result is returned
// (uniformly) in wave 0.  Lanes: max, rebase to the common reference, sums.
// Waves: the same over the per-wave results, read from LDS by wave 0.
__device__ inline Acc block_reduce(Acc a, float* lds, int T, int tid) {
  const float wm = wave_max(a.m);
  rebase(a, ref_of(wm));
  Acc w;
  w.m = wm;
  w.c = a.c;
  w.S = wave_sum(a.S);
  w.U = wave_sum(a.U);
  const int wave = tid >> 6, nw = T >> 6;
  if (nw == 1) return w;
  if ((tid & 63) == 0) {
    lds[wave] = w.m;
    lds[kMaxWaves + wave] = w.S;
    lds[2 * kMaxWaves + wave] = w.U;
  }
  __syncthreads();
  Acc r = acc_empty();
  if (wave == 0) {
    const int l = tid;
    Acc b = acc_empty();
    if (l < nw) {
      b.m = lds[l];
      b.c = ref_of(b.m);
      b.S = lds[kMaxWaves + l];
      b.U = lds[2 * kMaxWaves + l];
    }
    const float bm = lane_value(row16_max(b.m), 0);
    rebase(b, ref_of(bm));
    r.m = bm;
    r.c = b.c;
    r.S = lane_value(row16_sum(b.S), 0);
    r.U = lane_value(row16_sum(b.U), 0);
  }
  return r;
}

// lse about the exact max: m + ln2*(log2 S - d), d = m*log2e + c exactly.
__device__ inline float lse_of(const Acc& r) {
  const float d = fmaf(r.m, kLog2e, r.c);
  return r.S == 0.0f ? -INFINITY : r.m + kLn2 * (log2_hw(r.S) - d);
}
__device__ inline float entropy_of(const Acc& r) {
  return kLn2 * (log2_hw(r.S) - r.U / r.S);
}

// ---------------------------------------------------------------- kernels

struct FwdArgs {
  const char* logits;
  int64_t n_rows, width, row_bytes;   // width = vocab or chunk width
  int64_t vocab, vocab_offset;        // label range [0, vocab); chunk start
  const int64_t* labels;
  int64_t ignore_index;
  float* logprob;
  float* entropy;
  float* lse;
  bi_stats* stats;                    // chunk mode output
  int32_t* status_flag;
};

enum { kFull = 0, kChunk = 1 };

// ALIGNED: every row starts on a 4-byte boundary (checked on the host), so
// only the vector path is compiled in; otherwise each row picks its path.
template <int DT, int MODE, bool ALIGNED>
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(8)))
void fwd_kernel(FwdArgs p) {
  __shared__ float lds[3 * kMaxWaves];
  const int T = blockDim.x, tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
    const char* rp = p.logits + row * p.row_bytes;
    // the label's logit, loaded by thread 0 before the scan
    const int64_t y = p.labels[row];
    const bool ignored = y == p.ignore_index;
    const bool bad = !ignored && (y < 0 || y >= p.vocab);
    const int64_t local = y - p.vocab_offset;
    const bool inside = !ignored && !bad && local >= 0 && local < p.width;
    float zy = 0.0f;
    if (tid == 0 && inside) zy = Elt<DT>::load1(rp, local);

    Acc a = acc_empty();
    const RowSrc src = row_src(rp, p.width * (DT == BI_BF16 ? 2 : 4), T, tid);
    if (ALIGNED || (reinterpret_cast<uintptr_t>(rp) & 3u) == 0) {
      row_scan<DT, true>(a, src, p.width, T, tid);
    } else {
      row_scan<DT, false>(a, src, p.width, T, tid);
    }
    const Acc r = block_reduce(a, lds, T, tid);
    if (tid == 0) {
      if (bad && p.status_flag) atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
      if constexpr (MODE == kFull) {
        const float lse = lse_of(r);
        if (p.lse) p.lse[row] = lse;
        if (p.entropy) p.entropy[row] = entropy_of(r);
        if (p.logprob) p.logprob[row] = bad ? NAN : (ignored ? 0.0f : zy - lse);
      } else {
        // natural-units statistics about the exact max m
        const float d = fmaf(r.m, kLog2e, r.c);
        const float f = exp2_hw(-d);
        bi_stats s;
        s.max = r.m;
        s.sumexp = r.S == 0.0f ? 0.0f : r.S * f;
        s.sumexp_logit = r.S == 0.0f ? 0.0f : kLn2 * (fmaf(-d, r.S, r.U) * f);
        s.target = bad ? NAN : (inside ? zy : 0.0f);
        p.stats[row] = s;
      }
    }
    if (row + gridDim.x < p.n_rows) __syncthreads();   // lds reused by the next row
  }
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (v_cvt_pk_bf16_f32)
  const __bf16 a = __bf16(lo), b = __bf16(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Where one lane writes the gradients of its vectors: vector k*T + tid holds
// VEC values of GSIZE bytes each.  The 4-byte-aligned path uses non-temporal
// global_store_dwordx4 from a per-step base plus the lane's offset.  (Buffer
// stores with an SGPR offset are avoided on purpose: for those the compiler
// inserts no wait state before the data registers are overwritten, and on
// gfx950 the stored data was then observed to be corrupted.)
template <int GT, int VEC>
struct RowDst {
  static constexpr int kBytes = VEC * (GT == BI_BF16 ? 2 : 4);   // per vector
  char* row;
  uint32_t lane_off, step_bytes;

  __device__ RowDst(char* r, int T, int tid) {
    row = r;
    lane_off = uint32_t(tid) * kBytes;
    step_bytes = uint32_t(T) * kBytes;
  }

  template <bool VSTORE>
  __device__ inline void store(uint32_t k, const float* g) const {
    u32x4 w[kBytes / 16];
    if constexpr (GT == BI_BF16) {
      static_assert(VEC == 8, "bf16 gradients come from bf16 logits");
      w[0].x = pack_bf16x2(g[0], g[1]);
      w[0].y = pack_bf16x2(g[2], g[3]);
      w[0].z = pack_bf16x2(g[4], g[5]);
      w[0].w = pack_bf16x2(g[6], g[7]);
    } else {
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h) {
        w[h].x = __float_as_uint(g[4 * h + 0]);
        w[h].y = __float_as_uint(g[4 * h + 1]);
        w[h].z = __float_as_uint(g[4 * h + 2]);
        w[h].w = __float_as_uint(g[4 * h + 3]);
      }
    }
    if constexpr (VSTORE) {
      char* base = row + k * step_bytes;
#pragma unroll
      for (int h = 0; h < kBytes / 16; ++h) {
        u32x4_a4* q = reinterpret_cast<u32x4_a4*>(base + lane_off + 16u * h);
        if constexpr (BI_STORE_NT) __builtin_nontemporal_store(static_cast<u32x4_a4>(w[h]), q);
        else *q = w[h];
      }
    } else {
      uint16_t* q = reinterpret_cast<uint16_t*>(row + k * step_bytes + lane_off);
#pragma unroll
      for (int h = 0; h < kBytes / 16; ++h) {
        q[8 * h + 0] = uint16_t(w[h].x); q[8 * h + 1] = uint16_t(w[h].x >> 16);
        q[8 * h + 2] = uint16_t(w[h].y); q[8 * h + 3] = uint16_t(w[h].y >> 16);
        q[8 * h + 4] = uint16_t(w[h].z); q[8 * h + 5] = uint16_t(w[h].z >> 16);
        q[8 * h + 6] = uint16_t(w[h].w); q[8 * h + 7] = uint16_t(w[h].w >> 16);
      }
    }
  }

  __device__ inline void store1(int64_t j, float g) const {
    if constexpr (GT == BI_BF16) {
      const __bf16 b = __bf16(g);
      reinterpret_cast<uint16_t*>(row)[j] = __builtin_bit_cast(uint16_t, b);
    } else {
      reinterpret_cast<float*>(row)[j] = g;
    }
  }
};

// p = 2^((z - lse) * log2e): the subtraction first keeps the relative error
// of p small even for logits far from zero.
__device__ inline float prob(float z, float lse) { return exp2_hw((z - lse) * kLog2e); }

template <int VEC>
__device__ inline void grad_vec(const float* z, float lse, float w, float* g) {
#pragma unroll
  for (int k = 0; k < VEC; ++k) g[k] = w * prob(z[k], lse);
}

// the label column gets w * (p - 1)
template <int VEC>
__device__ inline void grad_label(const float* z, float lse, float w, int slot, float* g) {
#pragma unroll
  for (int k = 0; k < VEC; ++k)
    if (k == slot) g[k] = w * (prob(z[k], lse) - 1.0f);
}

struct BwdArgs {
  const char* logits;
  char* grad;
  int64_t n_rows, vocab, row_bytes, grad_row_bytes;
  const int64_t* labels;
  int64_t ignore_index;
  const float* lse;
  const float* weights;
  int32_t* status_flag;
};

template <int DT, int GT, bool VLOAD, bool VSTORE>
__device__ inline void bwd_vec(const RowDst<GT, Elt<DT>::VEC>& dst, uint32_t k, const u32x4& raw,
                               float lse, float w, uint32_t label_lane, int slot, int tid) {
  constexpr int VEC = Elt<DT>::VEC;
  float z[VEC], g[VEC];
  Elt<DT>::decode(raw, z);
  grad_vec<VEC>(z, lse, w, g);
  if (uint32_t(tid) == label_lane) grad_label<VEC>(z, lse, w, slot, g);
  dst.template store<VSTORE>(k, g);
}

// Vectors per lane per load group in the backward (the next group's loads
// are in flight while one is written).  The backward is elementwise, so this
// is pure pipelining and changes no result bit: for bf16 logits and bf16
// gradients in the kernels built for aligned rows (DEEP), 3 (24 elements) was
// the fastest depth that keeps the fused kernel within its 64 registers; the
// other kernels keep the rescale group's size.
template <int DT, int GT, bool DEEP>
constexpr int kBwdGroup =
    (DEEP && DT == BI_BF16 && GT == BI_BF16) ? 3 : kGroupElems / Elt<DT>::VEC;

template <int DT, int GT, bool VLOAD, bool VSTORE, int POL = kNonTemporal, bool REV = false,
          bool DEEP = false>
__device__ inline void bwd_row(const BwdArgs& p, const RowSrc& src,
                               const RowDst<GT, Elt<DT>::VEC>& dst, int64_t y, int kind,
                               float lse, float w, int T, int tid) {
  constexpr int VEC = Elt<DT>::VEC;
  constexpr int G = kBwdGroup<DT, GT, DEEP>;
  const int64_t width = p.vocab;
  const uint32_t nfull = uint32_t(width / VEC);
  const uint32_t nvec = uint32_t((width + VEC - 1) / VEC);
  const uint32_t full_steps = nfull / uint32_t(T);
  // the label's vector is yv = k*T + lane: lane = yv - k*T in step k
  const uint32_t yv = kind == 0 ? uint32_t(y / VEC) : 0xffffffffu;
  const int slot = int(y % VEC);

  if (kind != 0) {   // ignored rows: +0.0; bad labels: NaN; logits not read
    float g[VEC];
    const float fill = kind == 1 ? 0.0f : NAN;
#pragma unroll
    for (int k = 0; k < VEC; ++k) g[k] = fill;
    for (uint32_t k = 0; k < full_steps; ++k) dst.template store<VSTORE>(k, g);
    const uint32_t v = full_steps * uint32_t(T) + tid;
    if (v < nfull) dst.template store<VSTORE>(full_steps, g);
    else if (v == nfull)
      for (int64_t j = int64_t(v) * VEC; j < width; ++j) dst.store1(j, fill);
    return;
  }
  const uint32_t ngroups = full_steps / G;
  auto groups = [&] {
    pipelined_groups<DT, G, VLOAD, POL, REV>(src, ngroups, [&](const u32x4* buf, uint32_t g) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const uint32_t k = g * G + i;
        bwd_vec<DT, GT, VLOAD, VSTORE>(dst, k, buf[i], lse, w, yv - k * uint32_t(T), slot, tid);
      }
    });
  };
  auto rest = [&] {
    for (uint32_t k = ngroups * G; k < full_steps; ++k)
      bwd_vec<DT, GT, VLOAD, VSTORE>(dst, k, fetch<VLOAD, POL>(src, k), lse, w,
                                     yv - k * uint32_t(T), slot, tid);
    if (full_steps * uint32_t(T) < nvec) {
      const uint32_t k = full_steps, v = k * uint32_t(T) + tid;
      if (v < nfull) {
        bwd_vec<DT, GT, VLOAD, VSTORE>(dst, k, fetch<VLOAD, POL>(src, k), lse, w,
                                       yv - k * uint32_t(T), slot, tid);
      } else if (v == nfull) {
        for (int64_t j = int64_t(v) * VEC; j < width; ++j) {
          const float z = Elt<DT>::load1(src.row, j);
          dst.store1(j, j == y ? w * (prob(z, lse) - 1.0f) : w * prob(z, lse));
        }
      }
    }
  };
  if constexpr (REV) {
    rest();
    groups();
  } else {
    groups();
    rest();
  }
}

template <int DT, int GT, bool ALIGNED>
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(8)))
void bwd_kernel(BwdArgs p) {
  constexpr int VEC = Elt<DT>::VEC;
  const int T = blockDim.x, tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
    const char* rp = p.logits + row * p.row_bytes;
    char* gp = p.grad + row * p.grad_row_bytes;
    const int64_t y = p.labels[row];
    const int kind = y == p.ignore_index ? 1 : ((y < 0 || y >= p.vocab) ? 2 : 0);
    if (kind == 2 && tid == 0 && p.status_flag) atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
    const float lse = kind == 0 ? p.lse[row] : 0.0f;
    const float w = (kind == 0 && p.weights) ? p.weights[row] : 1.0f;
    const RowSrc src = row_src(rp, p.vocab * (DT == BI_BF16 ? 2 : 4), T, tid);
    const RowDst<GT, VEC> dst(gp, T, tid);
    const bool vload = ALIGNED || (reinterpret_cast<uintptr_t>(rp) & 3u) == 0;
    const bool vstore = ALIGNED || (reinterpret_cast<uintptr_t>(gp) & 3u) == 0;
    if (ALIGNED || (vload && vstore)) {
      bwd_row<DT, GT, true, true, kNonTemporal, false, ALIGNED>(p, src, dst, y, kind, lse, w,
                                                                 T, tid);
    } else if (vload) {
      bwd_row<DT, GT, true, false>(p, src, dst, y, kind, lse, w, T, tid);
    } else if (vstore) {
      bwd_row<DT, GT, false, true>(p, src, dst, y, kind, lse, w, T, tid);
    } else {
      bwd_row<DT, GT, false, false>(p, src, dst, y, kind, lse, w, T, tid);
    }
  }
}

// ------------------------------------------- backward as a sweep of pieces
//
// The backward is elementwise once lse is known, so it need not give a row to
// one workgroup: here workgroup b takes piece b % pieces (kSweepVecs
// consecutive 16-byte vectors, one per lane) of row b / pieces.  The pieces of
// consecutive rows follow each other in dispatch order, so the requests in
// flight stay in a narrow window of addresses that sweeps through the logits
// and the gradient, as a library elementwise kernel's do.  A plain copy of the
// 32,768 x 151,936 bf16 logits shaped this way moves 6.4 TB/s, against
// 5.0-5.1 TB/s for one 1,024-lane workgroup per row.  The arithmetic per
// element is bwd_vec's (and the ragged tail's is bwd_row's), so the bits are
// the row kernel's.
constexpr int kSweepVecs = 256;

template <int DT, int GT>
__global__ __launch_bounds__(kSweepVecs) void bwd_sweep_kernel(BwdArgs p, uint32_t pieces) {
  constexpr int VEC = Elt<DT>::VEC;
  const uint32_t row32 = blockIdx.x / pieces;
  const uint32_t piece = blockIdx.x - row32 * pieces;
  const int64_t row = row32;
  const int tid = threadIdx.x;
  const int64_t width = p.vocab;
  const uint32_t nfull = uint32_t(width / VEC);
  const uint32_t v = piece * uint32_t(kSweepVecs) + uint32_t(tid);   // the lane's vector
  const int64_t y = p.labels[row];
  const int kind = y == p.ignore_index ? 1 : ((y < 0 || y >= width) ? 2 : 0);
  if (kind == 2 && piece == 0 && tid == 0 && p.status_flag)
    atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
  const char* rp = p.logits + row * p.row_bytes;
  const RowDst<GT, VEC> dst(p.grad + row * p.grad_row_bytes, kSweepVecs, tid);
  if (kind != 0) {   // ignored rows: +0.0; bad labels: NaN; logits not read
    float g[VEC];
    const float fill = kind == 1 ? 0.0f : NAN;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g[e] = fill;
    if (v < nfull) dst.template store<true>(piece, g);
    else if (v == nfull)
      for (int64_t j = int64_t(v) * VEC; j < width; ++j) dst.store1(j, fill);
    return;
  }
  const float lse = p.lse[row];
  const float w = p.weights ? p.weights[row] : 1.0f;
  if (v < nfull) {
    const RowSrc src = row_src(rp, width * (DT == BI_BF16 ? 2 : 4), kSweepVecs, tid);
    bwd_vec<DT, GT, true, true>(dst, piece, fetch<true>(src, piece), lse, w,
                                uint32_t(y / VEC) - piece * uint32_t(kSweepVecs), int(y % VEC),
                                tid);
  } else if (v == nfull) {
    for (int64_t j = int64_t(v) * VEC; j < width; ++j) {
      const float z = Elt<DT>::load1(rp, j);
      dst.store1(j, j == y ? w * (prob(z, lse) - 1.0f) : w * prob(z, lse));
    }
  }
}

// ------------------------------------------- fused forward + backward
//
// One pass over each row when the per-token weight is known up front: the
// forward statistics and the gradient come from a single read of the logits
// (4 bytes per element at bf16/bf16 instead of 6 for the two calls).  The
// forward accumulates in exactly the order of row_scan and the gradient uses
// exactly bwd_vec's arithmetic, so every output is bit-identical to
// bi_logprob_fwd followed by bi_logprob_bwd.
//
// The second pass reads the row again; issued right after the first, it is
// served mostly by the caches, so HBM sees close to one read per element.
// (Keeping the whole row in registers instead needs ~76 VGPRs of a 128-VGPR
// budget at V = 151,936 bf16 and spilled.)

struct FusedArgs {
  const char* logits;
  char* grad;
  int64_t n_rows, vocab, row_bytes, grad_row_bytes;
  const int64_t* labels;
  int64_t ignore_index;
  const float* weights;
  float* logprob;
  float* entropy;
  float* lse;
  int32_t* status_flag;
  // clipped-ratio policy loss (POLICY kernels only)
  const float* old_logprob;
  const float* advantages;
  const float* loss_scale;
  float clip_low, clip_high;
  float* loss;
  float* weight_out;
};

// Weight of the clipped-ratio surrogate for one token (thread 0 only):
// r = exp(logprob - old), surrogate min(r A, clip(r, 1 - lo, 1 + hi) A), loss
// = -c * surrogate, weight = -d loss / d logprob = c A r where the unclipped
// term is the minimum (ties count as unclipped), else 0.
// The inputs of a row that the forward's finish needs besides the logits:
// its label logit and, for the policy loss, the behaviour logprob, the
// advantage and the loss scale.
struct RowScalars {
  float zy, old_logprob, advantage, scale;
};

__device__ inline float policy_weight(const FusedArgs& p, const RowScalars& in, float logprob,
                                      float* loss) {
  const float r = exp2_hw((logprob - in.old_logprob) * kLog2e);
  const float A = in.advantage;
  const float c = in.scale;
  const float rc = fminf(fmaxf(r, 1.0f - p.clip_low), 1.0f + p.clip_high);
  const bool unclipped = r * A <= rc * A;
  *loss = -c * (unclipped ? r * A : rc * A);
  return unclipped ? (c * A) * r : 0.0f;
}

// The first pass loads with the default cache policy so that the row stays in
// L2 / the Infinity Cache; the second pass re-reads it non-temporally, newest
// data first (its groups in reverse order).  Measured on the large bf16
// workload: 4.1 ms against 5.4-5.6 ms for the two separate calls.
#ifndef BI_FUSED_P1_POLICY
#define BI_FUSED_P1_POLICY 0
#endif
#ifndef BI_FUSED_P2_POLICY
#define BI_FUSED_P2_POLICY 2
#endif
#ifndef BI_FUSED_REVERSE
#define BI_FUSED_REVERSE 1
#endif

// The forward half of a fused row.  Every lane gets the lse and the weight of
// the gradient (the given one, or the policy-loss weight when POLICY).
// `scalars()` is called by thread 0 after the block reduction.
template <bool POLICY, typename Scalars>
__device__ inline void fused_finish(const FusedArgs& p, int64_t row, const Acc& a, float* lds,
                                    int T, int tid, bool ignored, bool bad, Scalars&& scalars,
                                    float* lse_out, float* w_out) {
  const Acc r = block_reduce(a, lds, T, tid);
  if (tid == 0) {
    const RowScalars in = scalars();
    const float lse = lse_of(r);
    const float lp = bad ? NAN : (ignored ? 0.0f : in.zy - lse);
    if (p.lse) p.lse[row] = lse;
    if (p.entropy) p.entropy[row] = entropy_of(r);
    if (p.logprob) p.logprob[row] = lp;
    if (bad && p.status_flag) atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
    lds[3 * kMaxWaves] = lse;
    if constexpr (POLICY) {
      float loss = bad ? NAN : 0.0f, w = bad ? NAN : 0.0f;
      if (!ignored && !bad) w = policy_weight(p, in, lp, &loss);
      if (p.loss) p.loss[row] = loss;
      if (p.weight_out) p.weight_out[row] = w;
      lds[3 * kMaxWaves + 1] = w;
    }
  }
  __syncthreads();
  *lse_out = lds[3 * kMaxWaves];
  if constexpr (POLICY) *w_out = lds[3 * kMaxWaves + 1];
}

// fused_finish with the row's inputs loaded by thread 0 when needed.
template <bool POLICY>
__device__ inline void fused_finish_forward(const FusedArgs& p, int64_t row, const Acc& a,
                                            float* lds, int T, int tid, float zy, bool ignored,
                                            bool bad, float* lse_out, float* w_out) {
  fused_finish<POLICY>(p, row, a, lds, T, tid, ignored, bad, [&] {
    RowScalars in{zy, 0.0f, 0.0f, 1.0f};
    if (POLICY && !ignored && !bad) {
      in.old_logprob = p.old_logprob[row];
      in.advantage = p.advantages[row];
      in.scale = p.loss_scale ? p.loss_scale[row] : 1.0f;
    }
    return in;
  }, lse_out, w_out);
}

template <int DT, int GT, bool ALIGNED, bool POLICY>
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(8)))
void fused_reread_kernel(FusedArgs p) {
  constexpr int VEC = Elt<DT>::VEC;
  __shared__ float lds[3 * kMaxWaves + 2];
  const int T = blockDim.x, tid = threadIdx.x;
  const int64_t width = p.vocab;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
    const char* rp = p.logits + row * p.row_bytes;
    char* gp = p.grad + row * p.grad_row_bytes;
    const int64_t y = p.labels[row];
    const bool ignored = y == p.ignore_index;
    const bool bad = !ignored && (y < 0 || y >= width);
    float zy = 0.0f;
    if (tid == 0 && !ignored && !bad) zy = Elt<DT>::load1(rp, y);
    float w = (!POLICY && !ignored && !bad && p.weights) ? p.weights[row] : 1.0f;
    const RowSrc src = row_src(rp, width * (DT == BI_BF16 ? 2 : 4), T, tid);
    const bool vload = ALIGNED || (reinterpret_cast<uintptr_t>(rp) & 3u) == 0;
    const bool vstore = ALIGNED || (reinterpret_cast<uintptr_t>(gp) & 3u) == 0;
    constexpr int P1 = BI_FUSED_P1_POLICY, P2 = BI_FUSED_P2_POLICY;
    constexpr bool REV = BI_FUSED_REVERSE;
    Acc a = acc_empty();
    if (vload) row_scan<DT, true, P1>(a, src, width, T, tid);
    else row_scan<DT, false, P1>(a, src, width, T, tid);
    float lse;
    fused_finish_forward<POLICY>(p, row, a, lds, T, tid, zy, ignored, bad, &lse, &w);
    const int kind = ignored ? 1 : (bad ? 2 : 0);
    const RowDst<GT, VEC> dst(gp, T, tid);
    BwdArgs b{p.logits, p.grad, p.n_rows, width, p.row_bytes, p.grad_row_bytes, p.labels,
              p.ignore_index, nullptr, nullptr, nullptr};
    if (ALIGNED || (vload && vstore))
      bwd_row<DT, GT, true, true, P2, REV, ALIGNED>(b, src, dst, y, kind, lse, w, T, tid);
    else if (vload)
      bwd_row<DT, GT, true, false, P2, REV>(b, src, dst, y, kind, lse, w, T, tid);
    else if (vstore)
      bwd_row<DT, GT, false, true, P2, REV>(b, src, dst, y, kind, lse, w, T, tid);
    else
      bwd_row<DT, GT, false, false, P2, REV>(b, src, dst, y, kind, lse, w, T, tid);
    if (row + gridDim.x < p.n_rows) __syncthreads();
  }
}

// ------------------------------------- fused forward + backward, row on chip
//
// bf16 rows of 131,073 .. 155,648 columns (a multiple of 8; the Qwen3
// vocabulary is one), 16-byte aligned: the geometry gives 1,024 lanes and
// FS full steps plus RAG ragged one per lane, 17 to 19 vectors, which the
// lane keeps in registers (4 VGPRs each).  One workgroup per compute unit
// walks rows b, b + grid, ...:
//  * pass 1 reduces the row from the registers in row_scan's exact order
//    (groups of two steps, then a single step, then the ragged step), and
//    block_reduce / lse / entropy are the row kernels' own, so every output
//    is bit-identical to bi_logprob_fwd;
//  * the row's first kPark vectors then move to LDS (each lane owns its slots
//    k * 1,024 + lane, so no barrier guards them) and the freed registers
//    take the next row's first kPark vectors, requested before the block
//    reduction so that they land during it;
//  * pass 2 writes the gradient (first the vectors in registers, then those
//    in LDS) with bwd_vec's arithmetic, bit-identical to bi_logprob_bwd, and
//    refills each register of steps kPark.. from the next row as soon as
//    its vector has been read.
// So each element is read from HBM once and the gradient written once, with
// the next row in flight while this one is reduced and written.  The kernel
// holds no value in scratch memory (about 120 VGPRs of 128).
//
// Waiting.  Vector memory operations complete in order, and stores count
// with loads, so a wait for one load also waits for everything issued before
// it.  The kernel is laid out so that no wait is for more than it needs:
// each refill load goes out before its vector's gradient store, the row's
// label, weight, policy inputs and label logit come a row ahead through the
// scalar data cache (counted by lgkmcnt instead), and the first row is
// peeled off the loop so that the loop's head is reached with the same
// operations in flight on both paths.

constexpr int kOnchipThreads = 1024;
constexpr int kPark = 9;   // vectors per lane parked in LDS: 9 x 16 KB per workgroup

// A pointer that is the same in every lane, held in SGPRs.
__device__ inline const char* sgpr_ptr(const char* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

// Scalar loads (s_load, into SGPRs) of a row's inputs: the kernel never
// writes them, and the scalar cache starts each dispatch invalidated.  The
// loads are inline assembly, and the value passes through the wait (also
// inline assembly), so no use can be scheduled before it.
__device__ inline uint32_t sload32(const void* q) {
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0" : "=s"(v) : "s"(q) : "memory");
  return v;
}
__device__ inline uint64_t sload64(const void* q) {
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0" : "=s"(v) : "s"(q) : "memory");
  return v;
}
__device__ inline void swait(uint32_t& v) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v) : : "memory");
}
__device__ inline void swait(uint64_t& v) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v) : : "memory");
}

// A row's label (int64 bits), weight, behaviour logprob, advantage and loss
// scale (fp32 bits).
struct OnchipRowIn {
  uint64_t y;
  uint32_t w, old_lp, adv, scale;
};

template <bool POLICY>
__device__ inline OnchipRowIn onchip_row_in(const FusedArgs& p, int64_t row) {
  OnchipRowIn in;
  in.y = sload64(p.labels + row);
  in.w = (!POLICY && p.weights) ? sload32(p.weights + row) : 0x3f800000u;
  in.old_lp = POLICY ? sload32(p.old_logprob + row) : 0u;
  in.adv = POLICY ? sload32(p.advantages + row) : 0u;
  in.scale = (POLICY && p.loss_scale) ? sload32(p.loss_scale + row) : 0x3f800000u;
  return in;
}

template <bool POLICY>
__device__ inline void onchip_row_wait(OnchipRowIn& in) {
  swait(in.y);
  swait(in.w);
  if constexpr (POLICY) {
    swait(in.old_lp);
    swait(in.adv);
    swait(in.scale);
  }
}

// The dword holding the bf16 logit of column y of a row that starts on a
// 4-byte boundary (its columns are y & ~1 and y | 1, both in the row when
// the width is even), and the logit itself.
__device__ inline uint32_t sload_label_logit(const char* row, int64_t y) {
  return sload32(row + (y & ~int64_t(1)) * 2);
}
__device__ inline float label_logit_of(uint32_t dword, int64_t y) {
  return __uint_as_float((y & 1) ? (dword & 0xffff0000u) : (dword << 16));
}

template <int GT, bool POLICY, int FS, bool RAG>
__global__ __launch_bounds__(kOnchipThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void fused_onchip_kernel(FusedArgs p) {
  constexpr int DT = BI_BF16, VEC = 8, T = kOnchipThreads;
  constexpr int NS = FS + (RAG ? 1 : 0);      // vectors per lane
  static_assert(NS > kPark && NS <= 19, "row held on chip");
  __shared__ __attribute__((aligned(1024))) u32x4 park[kPark * T];
  __shared__ float lds[3 * kMaxWaves + 2];
  const int tid = threadIdx.x;
  const int64_t width = p.vocab;
  const uint32_t nfull = uint32_t(width / VEC);            // width % 8 == 0: all vectors full
  const bool rag_lane = RAG && uint32_t(FS * T + tid) < nfull;   // holds a ragged-step vector
  const int row_bytes = int(width * 2);

  int64_t row = blockIdx.x;
  if (row >= p.n_rows) return;   // the whole workgroup together
  u32x4 r[NS];   // the row's vectors (steps 0 .. NS-1) in this lane

  // prologue: the first row's inputs, label logit and vectors (the ragged
  // step's vector is loaded by every lane: past the row's end the buffer
  // descriptor's range check returns zeros)
  OnchipRowIn in = onchip_row_in<POLICY>(p, row);
  onchip_row_wait<POLICY>(in);
  uint32_t zy_word = 0u;
  if (int64_t(in.y) >= 0 && int64_t(in.y) < width) {
    zy_word = sload_label_logit(p.logits + row * p.row_bytes, int64_t(in.y));
    swait(zy_word);
  }
  {
    RowSrc src = row_src(sgpr_ptr(p.logits + row * p.row_bytes), row_bytes, T, tid);
    asm volatile("" : "+s"(src.step_bytes));
#pragma unroll
    for (int k = 0; k < NS; ++k) r[k] = fetch<true>(src, uint32_t(k));
  }

  // One row; false after the workgroup's last row.  The loop runs it once
  // outside and then as its body, so that both ways into the loop's head
  // leave the same memory operations in flight (the compiler's waits at the
  // head are for the fewer of the two).
  auto row_step = [&]() -> bool {
    const int64_t next = row + gridDim.x;
    const bool has_next = next < p.n_rows;
    // this row's inputs are in scalar registers; the next row's are requested
    OnchipRowIn in_next = in;
    if (has_next) in_next = onchip_row_in<POLICY>(p, next);
    const int64_t y = int64_t(in.y);
    const bool ignored = y == p.ignore_index;
    const bool bad = !ignored && (y < 0 || y >= width);
    const int kind = ignored ? 1 : (bad ? 2 : 0);
    const float zy = kind == 0 ? label_logit_of(zy_word, y) : 0.0f;

    // pass 1: row_scan's order (groups of two steps, a single step, the
    // ragged step), one group at a time: a group's vectors are copied out of
    // their registers only after the previous group's terms are summed,
    // through a zero computed from the running sums.  Without that the
    // compiler decodes every group ahead and runs every group's max ahead of
    // the sums, keeping all their values live.
    Acc a = acc_empty();
    auto vec_after = [&](int k, const Acc& acc) -> u32x4 {
      uint32_t tok;
      asm volatile("v_and_b32 %0, 0, %1\n\tv_and_b32 %0, %0, %2"
                   : "=&v"(tok)
                   : "v"(acc.S), "v"(acc.U));
      u32x4 q = r[k];
      asm volatile("v_or_b32 %0, %0, %1" : "+v"(q.x) : "v"(tok));
      return q;
    };
#pragma unroll
    for (int g = 0; g < FS / 2; ++g) {
      float z[2 * VEC];
      const u32x4 v0 = vec_after(2 * g, a), v1 = vec_after(2 * g + 1, a);
      Elt<DT>::decode(v0, z);
      Elt<DT>::decode(v1, z + VEC);
      accumulate<VEC, 2>(a, z);
    }
    if constexpr (FS % 2 == 1) {
      float z[VEC];
      Elt<DT>::decode(vec_after(FS - 1, a), z);
      accumulate<VEC, 1>(a, z);
    }
    if constexpr (RAG) {
      // lanes past the row's end take -inf, which adds exactly nothing
      float z[VEC];
      Elt<DT>::decode(vec_after(FS, a), z);
#pragma unroll
      for (int e = 0; e < VEC; ++e) z[e] = rag_lane ? z[e] : -INFINITY;
      accumulate<VEC, 1>(a, z);
    }

    // the row's first kPark vectors move to LDS (this lane's slots), and the
    // registers they free take the next row's first kPark vectors, requested
    // now, before the block reduction: they are the first the next row's
    // pass 1 needs, and nothing issued later (this row's gradient stores)
    // has to land before them
    RowSrc nsrc = row_src(sgpr_ptr(p.logits + (has_next ? next : row) * p.row_bytes), row_bytes,
                          T, tid);
    asm volatile("" : "+s"(nsrc.step_bytes));
#pragma unroll
    for (int k = 0; k < kPark; ++k) park[k * T + tid] = r[k];
    // (after the last row these reload it: no branch around the loads, so
    // the compiler's count of what is in flight is the same on every path)
#pragma unroll
    for (int k = 0; k < kPark; ++k) r[k] = fetch<true>(nsrc, uint32_t(k));
    if (has_next) {
      // the next row's label has arrived: request its label logit
      onchip_row_wait<POLICY>(in_next);
      const int64_t yn = int64_t(in_next.y);
      if (yn >= 0 && yn < width) zy_word = sload_label_logit(p.logits + next * p.row_bytes, yn);
    }

    float lse, w = (!POLICY && kind == 0) ? __uint_as_float(in.w) : 1.0f;
    fused_finish<POLICY>(p, row, a, lds, T, tid, ignored, bad, [&] {
      return RowScalars{zy, __uint_as_float(in.old_lp), __uint_as_float(in.adv),
                        __uint_as_float(in.scale)};
    }, &lse, &w);

    // pass 2: the gradient of each vector: first those still in registers
    // (steps kPark ..), each register refilled from the next row as soon as
    // its vector is read, the load issued before the store; then those in
    // LDS (steps 0 .. kPark-1).  Memory operations complete in order, so the
    // next row's pass 1, waiting for a refill, also waits for the stores
    // issued before it: this order puts at most NS - kPark - 1 of them
    // there, and the LDS vectors' stores behind every load.
    // Every element is written as w * p (bwd_vec's arithmetic); the label's
    // element, w * (p - 1), is written over it afterwards by the lane that
    // holds it (one lane's stores to one address land in program order), so
    // the bits are bi_logprob_bwd's.  Ignored rows get +0.0 and bad labels
    // NaN, whatever their logits.
    const RowDst<GT, VEC> dst(p.grad + row * p.grad_row_bytes, T, tid);
    const bool live = kind == 0;
    const float fill = kind == 1 ? 0.0f : NAN;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int k = j < NS - kPark ? kPark + j : j - (NS - kPark);
      // decoded afresh (from a copy the compiler cannot see through), not
      // kept from pass 1
      u32x4 q = k < kPark ? park[k * T + tid] : r[k];
      asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
      float z[VEC], g[VEC];
      Elt<DT>::decode(q, z);
      grad_vec<VEC>(z, lse, w, g);
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[e] = live ? g[e] : fill;
      if (k >= kPark) {
        r[k] = fetch<true>(nsrc, uint32_t(k));
        __builtin_amdgcn_sched_barrier(0);   // the load goes out before the store
      }
      if (k < FS || rag_lane) dst.template store<true>(uint32_t(k), g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (live && uint32_t(tid) == uint32_t(y / VEC) % uint32_t(T))
      dst.store1(y, w * (prob(zy, lse) - 1.0f));

    if (!has_next) return false;
    swait(zy_word);
    in = in_next;
    row = next;
    __syncthreads();   // lds (the reduction's) is reused by the next row
    return true;
  };
  if (row_step())
    while (row_step()) {
    }
}

// ------------------------------------------------ several labels per row
//
// The generator side of trainer/generator parity: K token ids per row share
// one lse.  The scan, reduction and lse are exactly bi_logprob_fwd's, so the
// column that holds a row's label carries the same bits as bi_logprob_fwd.

struct MultiArgs {
  const char* logits;
  int64_t n_rows, vocab, row_bytes;
  const int64_t* labels;
  int64_t label_stride, k, ignore_index;
  float* logprob;            // [n_rows, k]
  float* entropy;
  float* lse;
  int32_t* status_flag;
};

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(8)))
void fwd_multi_kernel(MultiArgs p) {
  __shared__ float lds[3 * kMaxWaves + 1];
  const int T = blockDim.x, tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
    const char* rp = p.logits + row * p.row_bytes;
    const int64_t* yrow = p.labels + row * p.label_stride;
    // the first T label logits are fetched before the scan
    int64_t y0 = p.ignore_index;
    float z0 = 0.0f;
    if (tid < p.k) {
      y0 = yrow[tid];
      if (y0 != p.ignore_index && y0 >= 0 && y0 < p.vocab) z0 = Elt<DT>::load1(rp, y0);
    }
    Acc a = acc_empty();
    const RowSrc src = row_src(rp, p.vocab * (DT == BI_BF16 ? 2 : 4), T, tid);
    if (ALIGNED || (reinterpret_cast<uintptr_t>(rp) & 3u) == 0) {
      row_scan<DT, true>(a, src, p.vocab, T, tid);
    } else {
      row_scan<DT, false>(a, src, p.vocab, T, tid);
    }
    const Acc r = block_reduce(a, lds, T, tid);
    if (tid == 0) {
      const float l = lse_of(r);
      if (p.lse) p.lse[row] = l;
      if (p.entropy) p.entropy[row] = entropy_of(r);
      lds[3 * kMaxWaves] = l;
    }
    __syncthreads();
    const float lse = lds[3 * kMaxWaves];
    for (int64_t j = tid; j < p.k; j += T) {
      const int64_t y = j == tid ? y0 : yrow[j];
      const bool ignored = y == p.ignore_index;
      const bool bad = !ignored && (y < 0 || y >= p.vocab);
      float zy = j == tid ? z0 : 0.0f;
      if (j != tid && !ignored && !bad) zy = Elt<DT>::load1(rp, y);
      if (bad && p.status_flag) atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
      p.logprob[row * p.k + j] = bad ? NAN : (ignored ? 0.0f : zy - lse);
    }
    if (row + gridDim.x < p.n_rows) __syncthreads();
  }
}

// ------------------------------------ trainer-vs-generator difference metrics
//
// One workgroup: each lane sums its strided tokens in fp64, then a fixed tree
// over the lanes; out = (mean d, mean |d|, max |d|, fraction of tokens whose
// bits differ) with d = a - b over tokens whose label is not ignore_index.

constexpr int kDiffThreads = 1024;

__global__ __launch_bounds__(kDiffThreads) void diff_stats_kernel(
    const float* a, const float* b, const int64_t* labels, int64_t ignore_index, int64_t n,
    float* out) {
  __shared__ double sd[kDiffThreads], sa[kDiffThreads];
  __shared__ float sm[kDiffThreads];
  __shared__ int64_t sc[kDiffThreads], sx[kDiffThreads];
  const int tid = threadIdx.x;
  double d_sum = 0.0, a_sum = 0.0;
  float mx = 0.0f;
  int64_t cnt = 0, differ = 0;
  for (int64_t i = tid; i < n; i += kDiffThreads) {
    if (labels && labels[i] == ignore_index) continue;
    const float x = a[i], y = b[i];
    const double d = double(x) - double(y);
    d_sum += d;
    a_sum += fabs(d);
    const float ad = fabsf(x - y);
    mx = (ad > mx || ad != ad) ? ad : mx;   // NaN sticks
    cnt += 1;
    differ += __float_as_uint(x) != __float_as_uint(y);
  }
  sd[tid] = d_sum; sa[tid] = a_sum; sm[tid] = mx; sc[tid] = cnt; sx[tid] = differ;
  __syncthreads();
  for (int w = kDiffThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      sd[tid] += sd[tid + w];
      sa[tid] += sa[tid + w];
      const float o = sm[tid + w];
      sm[tid] = (o > sm[tid] || o != o) ? o : sm[tid];
      sc[tid] += sc[tid + w];
      sx[tid] += sx[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double c = double(sc[0]);
    out[0] = sc[0] ? float(sd[0] / c) : 0.0f;
    out[1] = sc[0] ? float(sa[0] / c) : 0.0f;
    out[2] = sc[0] ? sm[0] : 0.0f;
    out[3] = sc[0] ? float(double(sx[0]) / c) : 0.0f;
  }
}

// One thread per row, chunks in ascending order (natural units): the max
// first (exact, any order), then the sums about it, chunk 0, 1, 2, ...  The
// loads of eight chunks are issued ahead of their (in-order) arithmetic, and
// workgroups are one wave, so that 32,768 rows occupy 512 workgroups.
constexpr int kCombineThreads = 64;
constexpr int kCombineAhead = 8;

__device__ inline void combine_step(const bi_stats& s, float M, float& S, float& U, float& t) {
  t += s.target;
  if (s.sumexp > 0.0f) {
    const float gap = s.max - M;
    const float a = exp2_hw(gap * kLog2e);
    S = fmaf(a, s.sumexp, S);
    U = fmaf(a, fmaf(gap, s.sumexp, s.sumexp_logit), U);
  } else if (!(s.sumexp == 0.0f)) {   // NaN statistics propagate
    S = NAN;
  }
}

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const bi_stats* stats, int64_t n_chunks, int64_t n_rows, const int64_t* labels,
    int64_t ignore_index, float* logprob, float* entropy, float* lse_out) {
  const int64_t row = int64_t(blockIdx.x) * kCombineThreads + threadIdx.x;
  if (row >= n_rows) return;
  const bi_stats* s = stats + row;   // chunk c at s[c * n_rows]
  float M = -INFINITY;
  int64_t c = 0;
  for (; c + kCombineAhead <= n_chunks; c += kCombineAhead) {
    float mx[kCombineAhead];
#pragma unroll
    for (int k = 0; k < kCombineAhead; ++k) mx[k] = s[(c + k) * n_rows].max;
#pragma unroll
    for (int k = 0; k < kCombineAhead; ++k) M = fmaxf(M, mx[k]);
  }
  for (; c < n_chunks; ++c) M = fmaxf(M, s[c * n_rows].max);
  float S = 0.0f, U = 0.0f, t = 0.0f;
  for (c = 0; c + kCombineAhead <= n_chunks; c += kCombineAhead) {
    bi_stats v[kCombineAhead];
#pragma unroll
    for (int k = 0; k < kCombineAhead; ++k) v[k] = s[(c + k) * n_rows];
#pragma unroll
    for (int k = 0; k < kCombineAhead; ++k) combine_step(v[k], M, S, U, t);
  }
  for (; c < n_chunks; ++c) combine_step(s[c * n_rows], M, S, U, t);
  const float lnS = kLn2 * log2_hw(S);
  const float lse = S == 0.0f ? -INFINITY : M + lnS;
  const int64_t y = labels[row];
  if (lse_out) lse_out[row] = lse;
  if (entropy) entropy[row] = lnS - U / S;
  if (logprob) logprob[row] = y == ignore_index ? 0.0f : t - lse;
}

// ------------------------------------------------------------- host side

}  // namespace

namespace bi_internal {

namespace {
thread_local char g_err[512];
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return BI_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BI_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

const char* last_error() { return g_err; }

}  // namespace bi_internal

namespace {

size_t elem_size(int dt) { return dt == BI_BF16 ? 2 : 4; }

int check_dtype(int dt, const char* what) {
  if (dt != BI_F32 && dt != BI_BF16) return fail(BI_ERR_DTYPE, "%s: unknown dtype %d", what, dt);
  return BI_OK;
}

// One workgroup per row, at most as many as keep the dispatch's size in
// work-items within 32 bits (the kernels loop over the rows beyond).
unsigned grid_for(int64_t n_rows, int threads) {
  const int64_t cap = int64_t(0xffffffffu) / threads;
  return unsigned(n_rows < cap ? n_rows : cap);
}

// every row of a [n_rows, row_bytes] array starting at p is 4-byte aligned
bool rows_dword_aligned(const void* p, int64_t row_bytes) {
  return aligned(p, 4) && (row_bytes % 4) == 0;
}

template <int DT, int MODE>
void launch_fwd(const FwdArgs& a, int threads, hipStream_t s) {
  const dim3 grid(grid_for(a.n_rows, threads)), block(threads);
  if (DT == BI_F32 || rows_dword_aligned(a.logits, a.row_bytes))
    hipLaunchKernelGGL((fwd_kernel<DT, MODE, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<DT, MODE, false>), grid, block, 0, s, a);
}

template <int DT, int GT>
void launch_bwd(const BwdArgs& a, int threads, hipStream_t s) {
  const bool dword_rows =
      rows_dword_aligned(a.logits, a.row_bytes) && rows_dword_aligned(a.grad, a.grad_row_bytes);
  // rows of at least 16 pieces on 4-byte boundaries: the sweep of pieces
  constexpr int VEC = Elt<DT>::VEC;
  const int64_t pieces = ((a.vocab + VEC - 1) / VEC + kSweepVecs - 1) / kSweepVecs;
  if (dword_rows && pieces >= 16 &&
      a.n_rows * pieces <= int64_t(0xffffffffu) / kSweepVecs) {
    hipLaunchKernelGGL((bwd_sweep_kernel<DT, GT>), dim3(unsigned(a.n_rows * pieces)),
                       dim3(kSweepVecs), 0, s, a, uint32_t(pieces));
    return;
  }
  const dim3 grid(grid_for(a.n_rows, threads)), block(threads);
  if (dword_rows)
    hipLaunchKernelGGL((bwd_kernel<DT, GT, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((bwd_kernel<DT, GT, false>), grid, block, 0, s, a);
}

#ifndef BI_FUSED_ONCHIP
#define BI_FUSED_ONCHIP 1
#endif

// Compute units of the current device (cached per device).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The row-on-chip fused kernel for bf16 rows of 1,024-lane geometry whose
// vectors fit the registers (17..19 per lane), every vector full, logits rows
// 16-byte aligned and gradient rows 4-byte aligned; false: the re-read kernel.
template <bool POLICY>
bool launch_fused_onchip(const FusedArgs& a, int grad_dtype, hipStream_t s) {
  if (!BI_FUSED_ONCHIP) return false;
  const int64_t nvec = a.vocab / 8;
  if (a.vocab % 8 != 0 || nvec <= int64_t(16) * kOnchipThreads ||
      nvec > int64_t(19) * kOnchipThreads)
    return false;
  if (!aligned(a.logits, 16) || a.row_bytes % 16 != 0 ||
      !rows_dword_aligned(a.grad, a.grad_row_bytes))
    return false;
  const int fs = int(nvec / kOnchipThreads);
  const bool rag = nvec % kOnchipThreads != 0;
  const int64_t cus = compute_units();
  const dim3 grid(unsigned(a.n_rows < cus ? a.n_rows : cus)), block(kOnchipThreads);
#define BI_ONCHIP(GT, FS, RAG) \
  hipLaunchKernelGGL((fused_onchip_kernel<GT, POLICY, FS, RAG>), grid, block, 0, s, a)
#define BI_ONCHIP_GT(FS, RAG)                                   \
  do {                                                          \
    if (grad_dtype == BI_BF16) BI_ONCHIP(BI_BF16, FS, RAG);     \
    else BI_ONCHIP(BI_F32, FS, RAG);                            \
  } while (0)
  if (fs == 16 && rag) BI_ONCHIP_GT(16, true);
  else if (fs == 17 && !rag) BI_ONCHIP_GT(17, false);
  else if (fs == 17) BI_ONCHIP_GT(17, true);
  else if (fs == 18 && !rag) BI_ONCHIP_GT(18, false);
  else if (fs == 18) BI_ONCHIP_GT(18, true);
  else BI_ONCHIP_GT(19, false);
#undef BI_ONCHIP_GT
#undef BI_ONCHIP
  return true;
}

template <bool POLICY>
int launch_fused(const char* fn, FusedArgs a, int dtype, int grad_dtype, int64_t row_stride,
                 int64_t grad_row_stride, bi_stream_t stream) {
  if (int r = check_dtype(dtype, fn)) return r;
  if (int r = check_dtype(grad_dtype, fn)) return r;
  if (dtype == BI_F32 && grad_dtype == BI_BF16)
    return fail(BI_ERR_DTYPE, "%s: fp32 logits with a bf16 gradient are not supported", fn);
  if (a.n_rows < 0) return fail(BI_ERR_SHAPE, "%s: n_rows %lld < 0", fn, (long long)a.n_rows);
  if (a.vocab < 1 || a.vocab >= kMaxWidth)
    return fail(BI_ERR_SHAPE, "%s: vocab %lld outside [1, 2^29)", fn, (long long)a.vocab);
  if (row_stride < a.vocab || grad_row_stride < a.vocab)
    return fail(BI_ERR_SHAPE, "%s: row strides (%lld, %lld) must be >= vocab %lld", fn,
                (long long)row_stride, (long long)grad_row_stride, (long long)a.vocab);
  if (a.n_rows == 0) return ok();
  if (!a.logits || !a.labels || !a.grad)
    return fail(BI_ERR_NULL, "%s: logits, labels and grad are required", fn);
  if (!aligned(a.logits, elem_size(dtype)) || !aligned(a.grad, elem_size(grad_dtype)) ||
      !aligned(a.labels, 8) || !aligned(a.weights, 4) || !aligned(a.logprob, 4) ||
      !aligned(a.entropy, 4) || !aligned(a.lse, 4) || !aligned(a.status_flag, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  a.row_bytes = row_stride * int64_t(elem_size(dtype));
  a.grad_row_bytes = grad_row_stride * int64_t(elem_size(grad_dtype));
  {
    // the gradient is written while other rows' logits are still to be read
    const uintptr_t l0 = reinterpret_cast<uintptr_t>(a.logits), g0 = reinterpret_cast<uintptr_t>(a.grad);
    const uintptr_t l1 = l0 + uintptr_t((a.n_rows - 1) * a.row_bytes + a.vocab * int64_t(elem_size(dtype)));
    const uintptr_t g1 = g0 + uintptr_t((a.n_rows - 1) * a.grad_row_bytes +
                                        a.vocab * int64_t(elem_size(grad_dtype)));
    if (l0 < g1 && g0 < l1)
      return fail(BI_ERR_SHAPE, "%s: grad overlaps the logits (their byte ranges must be disjoint)",
                  fn);
  }
  const Geometry g = row_geometry(dtype, a.vocab);
  const bool all_aligned = rows_dword_aligned(a.logits, a.row_bytes) &&
                           rows_dword_aligned(a.grad, a.grad_row_bytes);
  const dim3 grid(grid_for(a.n_rows, g.threads)), block(g.threads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BI_BF16 && g.threads == kOnchipThreads &&
      launch_fused_onchip<POLICY>(a, grad_dtype, s))
    return launched(fn);
#define BI_FUSED_LAUNCH(DT, GT)                                                              \
  do {                                                                                       \
    if (all_aligned)                                                                         \
      hipLaunchKernelGGL((fused_reread_kernel<DT, GT, true, POLICY>), grid, block, 0, s, a); \
    else                                                                                     \
      hipLaunchKernelGGL((fused_reread_kernel<DT, GT, false, POLICY>), grid, block, 0, s, a);\
  } while (0)
  if (dtype == BI_BF16 && grad_dtype == BI_BF16) BI_FUSED_LAUNCH(BI_BF16, BI_BF16);
  else if (dtype == BI_BF16) BI_FUSED_LAUNCH(BI_BF16, BI_F32);
  else BI_FUSED_LAUNCH(BI_F32, BI_F32);
#undef BI_FUSED_LAUNCH
  return launched(fn);
}

}  // namespace

extern "C" {

const char* bi_status_string(int status) {
  switch (status) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE: bad size, stride, vocabulary size or offset";
    case BI_ERR_DTYPE: return "BI_ERR_DTYPE: unknown or unsupported dtype";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN: pointer not aligned to its element size";
    case BI_ERR_LAUNCH: return "BI_ERR_LAUNCH: HIP launch failed";
    default: return "unknown status";
  }
}

const char* bi_last_error(void) { return last_error(); }

int bi_row_geometry(int dtype, int64_t width, int* threads, int* elems_per_load,
                    int* loads_per_group) {
  if (int r = check_dtype(dtype, "bi_row_geometry")) return r;
  if (width < 1 || width >= kMaxWidth) return fail(BI_ERR_SHAPE, "bi_row_geometry: width %lld", (long long)width);
  const Geometry g = row_geometry(dtype, width);
  if (threads) *threads = g.threads;
  if (elems_per_load) *elems_per_load = g.vec;
  if (loads_per_group) *loads_per_group = g.group;
  return ok();
}

int bi_logprob_fwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                   int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                   float* logprob, float* entropy, float* lse, int32_t* status_flag,
                   bi_stream_t stream) {
  const char* fn = "bi_logprob_fwd";
  if (int r = check_dtype(dtype, fn)) return r;
  if (n_rows < 0) return fail(BI_ERR_SHAPE, "%s: n_rows %lld < 0", fn, (long long)n_rows);
  if (vocab < 1 || vocab >= kMaxWidth)
    return fail(BI_ERR_SHAPE, "%s: vocab %lld outside [1, 2^29)", fn, (long long)vocab);
  if (row_stride < vocab)
    return fail(BI_ERR_SHAPE, "%s: row_stride %lld < vocab %lld", fn, (long long)row_stride, (long long)vocab);
  if (n_rows == 0) return ok();
  if (!logits || !labels) return fail(BI_ERR_NULL, "%s: logits and labels are required", fn);
  if (!logprob && !entropy && !lse) return fail(BI_ERR_NULL, "%s: no output requested", fn);
  if (!aligned(logits, elem_size(dtype)) || !aligned(labels, 8) || !aligned(logprob, 4) ||
      !aligned(entropy, 4) || !aligned(lse, 4) || !aligned(status_flag, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  FwdArgs a{static_cast<const char*>(logits), n_rows, vocab, row_stride * int64_t(elem_size(dtype)),
            vocab, 0, labels, ignore_index, logprob, entropy, lse, nullptr, status_flag};
  const Geometry g = row_geometry(dtype, vocab);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BI_BF16) launch_fwd<BI_BF16, kFull>(a, g.threads, s);
  else launch_fwd<BI_F32, kFull>(a, g.threads, s);
  return launched(fn);
}

int bi_vocab_chunk_stats(const void* logits_chunk, int dtype, int64_t n_rows,
                         int64_t chunk_width, int64_t row_stride, int64_t vocab_offset,
                         int64_t vocab, const int64_t* labels, int64_t ignore_index,
                         bi_stats* stats, int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_vocab_chunk_stats";
  if (int r = check_dtype(dtype, fn)) return r;
  if (n_rows < 0) return fail(BI_ERR_SHAPE, "%s: n_rows %lld < 0", fn, (long long)n_rows);
  if (vocab < 1 || vocab >= kMaxWidth)
    return fail(BI_ERR_SHAPE,
                "%s: the global vocabulary size is required (got %lld); it must lie in [1, 2^29)",
                fn, (long long)vocab);
  if (chunk_width < 1 || vocab_offset < 0 || vocab_offset + chunk_width > vocab)
    return fail(BI_ERR_SHAPE, "%s: chunk [%lld, %lld) outside the vocabulary [0, %lld)", fn,
                (long long)vocab_offset, (long long)(vocab_offset + chunk_width), (long long)vocab);
  if (row_stride < chunk_width)
    return fail(BI_ERR_SHAPE, "%s: row_stride %lld < chunk_width %lld", fn, (long long)row_stride,
                (long long)chunk_width);
  if (n_rows == 0) return ok();
  if (!logits_chunk || !labels || !stats) return fail(BI_ERR_NULL, "%s: logits, labels and stats are required", fn);
  if (!aligned(logits_chunk, elem_size(dtype)) || !aligned(labels, 8) || !aligned(stats, 4) ||
      !aligned(status_flag, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  FwdArgs a{static_cast<const char*>(logits_chunk), n_rows, chunk_width,
            row_stride * int64_t(elem_size(dtype)), vocab, vocab_offset, labels, ignore_index,
            nullptr, nullptr, nullptr, stats, status_flag};
  const Geometry g = row_geometry(dtype, chunk_width);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BI_BF16) launch_fwd<BI_BF16, kChunk>(a, g.threads, s);
  else launch_fwd<BI_F32, kChunk>(a, g.threads, s);
  return launched(fn);
}

int bi_logprob_bwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                   int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                   const float* lse, const float* weights, void* grad, int grad_dtype,
                   int64_t grad_row_stride, int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_logprob_bwd";
  if (int r = check_dtype(dtype, fn)) return r;
  if (int r = check_dtype(grad_dtype, fn)) return r;
  if (dtype == BI_F32 && grad_dtype == BI_BF16)
    return fail(BI_ERR_DTYPE, "%s: fp32 logits with a bf16 gradient are not supported", fn);
  if (n_rows < 0) return fail(BI_ERR_SHAPE, "%s: n_rows %lld < 0", fn, (long long)n_rows);
  if (vocab < 1 || vocab >= kMaxWidth)
    return fail(BI_ERR_SHAPE, "%s: vocab %lld outside [1, 2^29)", fn, (long long)vocab);
  if (row_stride < vocab || grad_row_stride < vocab)
    return fail(BI_ERR_SHAPE, "%s: row strides (%lld, %lld) must be >= vocab %lld", fn,
                (long long)row_stride, (long long)grad_row_stride, (long long)vocab);
  if (n_rows == 0) return ok();
  if (!logits || !labels || !lse || !grad)
    return fail(BI_ERR_NULL, "%s: logits, labels, lse and grad are required", fn);
  if (!aligned(logits, elem_size(dtype)) || !aligned(grad, elem_size(grad_dtype)) ||
      !aligned(labels, 8) || !aligned(lse, 4) || !aligned(weights, 4) || !aligned(status_flag, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  BwdArgs a{static_cast<const char*>(logits), static_cast<char*>(grad), n_rows, vocab,
            row_stride * int64_t(elem_size(dtype)), grad_row_stride * int64_t(elem_size(grad_dtype)),
            labels, ignore_index, lse, weights, status_flag};
  const Geometry g = row_geometry(dtype, vocab);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BI_BF16 && grad_dtype == BI_BF16) launch_bwd<BI_BF16, BI_BF16>(a, g.threads, s);
  else if (dtype == BI_BF16) launch_bwd<BI_BF16, BI_F32>(a, g.threads, s);
  else launch_bwd<BI_F32, BI_F32>(a, g.threads, s);
  return launched(fn);
}

int bi_logprob_fwd_bwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                       int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                       const float* weights, float* logprob, float* entropy, float* lse,
                       void* grad, int grad_dtype, int64_t grad_row_stride,
                       int32_t* status_flag, bi_stream_t stream) {
  FusedArgs a{static_cast<const char*>(logits), static_cast<char*>(grad), n_rows, vocab,
              0, 0, labels, ignore_index, weights, logprob, entropy, lse, status_flag,
              nullptr, nullptr, nullptr, 0.0f, 0.0f, nullptr, nullptr};
  return launch_fused<false>("bi_logprob_fwd_bwd", a, dtype, grad_dtype, row_stride,
                             grad_row_stride, stream);
}

int bi_policy_loss_fwd_bwd(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                           int64_t row_stride, const int64_t* labels, int64_t ignore_index,
                           const float* old_logprob, const float* advantages,
                           const float* loss_scale, float clip_low, float clip_high,
                           float* logprob, float* entropy, float* lse, float* loss,
                           float* weight, void* grad, int grad_dtype, int64_t grad_row_stride,
                           int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_policy_loss_fwd_bwd";
  if (!(clip_low >= 0.0f && clip_low < 1.0f) || !(clip_high >= 0.0f && clip_high < 1e30f))
    return fail(BI_ERR_SHAPE, "%s: clip bounds must satisfy 0 <= clip_low < 1, 0 <= clip_high",
                fn);
  if (n_rows > 0 && (!old_logprob || !advantages))
    return fail(BI_ERR_NULL, "%s: old_logprob and advantages are required", fn);
  if (!aligned(old_logprob, 4) || !aligned(advantages, 4) || !aligned(loss_scale, 4) ||
      !aligned(loss, 4) || !aligned(weight, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  FusedArgs a{static_cast<const char*>(logits), static_cast<char*>(grad), n_rows, vocab,
              0, 0, labels, ignore_index, nullptr, logprob, entropy, lse, status_flag,
              old_logprob, advantages, loss_scale, clip_low, clip_high, loss, weight};
  return launch_fused<true>(fn, a, dtype, grad_dtype, row_stride, grad_row_stride, stream);
}

int bi_logprob_fwd_multi(const void* logits, int dtype, int64_t n_rows, int64_t vocab,
                         int64_t row_stride, const int64_t* labels, int64_t label_stride,
                         int64_t k, int64_t ignore_index, float* logprob, float* entropy,
                         float* lse, int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_logprob_fwd_multi";
  if (int r = check_dtype(dtype, fn)) return r;
  if (n_rows < 0) return fail(BI_ERR_SHAPE, "%s: n_rows %lld < 0", fn, (long long)n_rows);
  if (vocab < 1 || vocab >= kMaxWidth)
    return fail(BI_ERR_SHAPE, "%s: vocab %lld outside [1, 2^29)", fn, (long long)vocab);
  if (row_stride < vocab)
    return fail(BI_ERR_SHAPE, "%s: row_stride %lld < vocab %lld", fn, (long long)row_stride,
                (long long)vocab);
  if (k < 1 || label_stride < k)
    return fail(BI_ERR_SHAPE, "%s: need 1 <= k <= label_stride (k %lld, stride %lld)", fn,
                (long long)k, (long long)label_stride);
  if (n_rows == 0) return ok();
  if (!logits || !labels || !logprob)
    return fail(BI_ERR_NULL, "%s: logits, labels and logprob are required", fn);
  if (!aligned(logits, elem_size(dtype)) || !aligned(labels, 8) || !aligned(logprob, 4) ||
      !aligned(entropy, 4) || !aligned(lse, 4) || !aligned(status_flag, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  MultiArgs a{static_cast<const char*>(logits), n_rows, vocab, row_stride * int64_t(elem_size(dtype)),
              labels, label_stride, k, ignore_index, logprob, entropy, lse, status_flag};
  const Geometry g = row_geometry(dtype, vocab);
  const dim3 grid(grid_for(n_rows, g.threads)), block(g.threads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool al = dtype == BI_F32 || rows_dword_aligned(logits, a.row_bytes);
  if (dtype == BI_BF16) {
    if (al) hipLaunchKernelGGL((fwd_multi_kernel<BI_BF16, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_multi_kernel<BI_BF16, false>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((fwd_multi_kernel<BI_F32, true>), grid, block, 0, s, a);
  }
  return launched(fn);
}

int bi_logprob_diff_stats(const float* a, const float* b, const int64_t* labels,
                          int64_t ignore_index, int64_t n, float* out, bi_stream_t stream) {
  const char* fn = "bi_logprob_diff_stats";
  if (n < 0) return fail(BI_ERR_SHAPE, "%s: n %lld < 0", fn, (long long)n);
  if (!out) return fail(BI_ERR_NULL, "%s: out is required", fn);
  if (n > 0 && (!a || !b)) return fail(BI_ERR_NULL, "%s: a and b are required", fn);
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(labels, 8) || !aligned(out, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  hipLaunchKernelGGL(diff_stats_kernel, dim3(1), dim3(kDiffThreads), 0,
                     static_cast<hipStream_t>(stream), a, b, labels, ignore_index, n, out);
  return launched(fn);
}

int bi_stats_combine(const bi_stats* stats, int64_t n_chunks, int64_t n_rows,
                     const int64_t* labels, int64_t ignore_index, float* logprob,
                     float* entropy, float* lse, bi_stream_t stream) {
  const char* fn = "bi_stats_combine";
  if (n_chunks < 1) return fail(BI_ERR_SHAPE, "%s: n_chunks %lld < 1", fn, (long long)n_chunks);
  if (n_rows < 0) return fail(BI_ERR_SHAPE, "%s: n_rows %lld < 0", fn, (long long)n_rows);
  if (n_rows == 0) return ok();
  if (!stats || !labels) return fail(BI_ERR_NULL, "%s: stats and labels are required", fn);
  if (!logprob && !entropy && !lse) return fail(BI_ERR_NULL, "%s: no output requested", fn);
  if (!aligned(stats, 4) || !aligned(labels, 8) || !aligned(logprob, 4) || !aligned(entropy, 4) ||
      !aligned(lse, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  const int64_t blocks = (n_rows + kCombineThreads - 1) / kCombineThreads;
  if (blocks > 0x7fffffff) return fail(BI_ERR_SHAPE, "%s: too many rows", fn);
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(blocks)), dim3(kCombineThreads), 0,
                     static_cast<hipStream_t>(stream), stats, n_chunks, n_rows, labels,
                     ignore_index, logprob, entropy, lse);
  return launched(fn);
}

}  // extern "C"
