// bi_ceilings.hip - two plain streaming kernels that measure the HBM ceilings
// the row kernels are judged against, in the same run: a read-only stream and
// a copy.  They compute nothing of the method; the benchmark times them over
// the same tensors as the row kernels (libbi_ceilings.so, not part of the
// library's C ABI in include/bi_logprob.h).
//
//  * read: 256-lane workgroups, four 16-byte non-temporal loads per lane in
//    flight (16 KB per workgroup, one pass, no loop); the loaded words are
//    XOR-folded and written only if the fold equals a fixed constant, so the
//    loads cannot be dropped while nearly nothing is stored.
//  * copy: 256-lane workgroups, one 16-byte non-temporal load and store per
//    lane (the fastest plain copy pattern found on this chip).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kReadDepth = 4;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                         int64_t n_vec, uint32_t* sink) {
  const int64_t base = int64_t(blockIdx.x) * (kThreads * kReadDepth) + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (base + (kReadDepth - 1) * kThreads < n_vec) {
    u32x4 v[kReadDepth];
#pragma unroll
    for (int k = 0; k < kReadDepth; ++k) v[k] = __builtin_nontemporal_load(src + base + k * kThreads);
#pragma unroll
    for (int k = 0; k < kReadDepth; ++k) acc ^= v[k];
  } else {
    for (int k = 0; k < kReadDepth; ++k)
      if (base + k * kThreads < n_vec) acc ^= __builtin_nontemporal_load(src + base + k * kThreads);
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9e3779b9u) sink[0] = x;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n_vec) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n_vec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

bool ok_ptr(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from `src`; `sink` is a device word that is
// written only when the XOR of everything read equals a fixed constant.
// Returns 0, -1 for bad arguments, or the HIP error code of the launch.
__attribute__((visibility("default"))) int bi_ceiling_read(const void* src, int64_t bytes,
                                                           void* sink, void* stream) {
  if (!ok_ptr(src) || !sink || bytes < 0 || bytes % 16) return -1;
  const int64_t n_vec = bytes / 16;
  const int64_t blocks = (n_vec + kThreads * kReadDepth - 1) / (kThreads * kReadDepth);
  if (blocks == 0) return 0;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n_vec,
                     static_cast<uint32_t*>(sink));
  return int(hipGetLastError());
}

// Copy `bytes` (a multiple of 16) from `src` to `dst`.
__attribute__((visibility("default"))) int bi_ceiling_copy(const void* src, void* dst,
                                                           int64_t bytes, void* stream) {
  if (!ok_ptr(src) || !ok_ptr(dst) || bytes < 0 || bytes % 16) return -1;
  const int64_t n_vec = bytes / 16;
  const int64_t blocks = (n_vec + kThreads - 1) / kThreads;
  if (blocks == 0) return 0;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n_vec);
  return int(hipGetLastError());
}

}  // extern "C"
