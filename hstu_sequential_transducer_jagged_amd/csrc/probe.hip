// Measurement probes for gfx950 (libhstu_probe.so): the bf16 matrix-core
// rate with no memory traffic, the HBM rate of a streaming copy, and the
// shader clock under matrix-core load. They are not part of the layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four independent accumulator chains per wave: a chain's next MFMA depends
// on its previous one, and four in rotation cover that dependency, so each
// wave issues back to back.
__global__ __launch_bounds__(HSTU_PROBE_MFMA_THREADS) void mfma_loop_kernel(float* sink, int64_t* clocks,
                                                                            int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + i) & 15));
    b[i] = static_cast<__bf16>(1e-3f * static_cast<float>(i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  // the loop's results are read before the end stamps
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  __syncthreads();
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (s == -1.0f) sink[threadIdx.x] = s;   // never true: keeps the chains live
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

constexpr int kCopyThreads = 256;
constexpr int kCopyVec = 4;   // 16-byte vectors per thread

// One pass, no loop: workgroup g copies the contiguous 16 KB chunk g, each
// thread four 16-byte vectors 4 KB apart, so that every load and store
// instruction of a workgroup covers 4 KB of consecutive memory.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const uint4* __restrict__ src,
                                                            uint4* __restrict__ dst, int64_t n) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kCopyThreads * kCopyVec) + threadIdx.x;
  uint4 v[kCopyVec];
#pragma unroll
  for (int k = 0; k < kCopyVec; ++k) {
    const int64_t i = base + k * kCopyThreads;
    if (i < n) v[k] = src[i];
  }
#pragma unroll
  for (int k = 0; k < kCopyVec; ++k) {
    const int64_t i = base + k * kCopyThreads;
    if (i < n) dst[i] = v[k];
  }
}

}  // namespace

extern "C" int hstu_probe_mfma_bf16(int num_groups, int iters, float* sink, int64_t* clocks, void* stream) {
  if (num_groups < 1 || iters < 1 || iters > (1 << 24) || !sink || !clocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(num_groups), dim3(HSTU_PROBE_MFMA_THREADS), 0,
                     static_cast<hipStream_t>(stream), sink, clocks, iters);
  return hipGetLastError();
}

extern "C" int hstu_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return hipErrorInvalidValue;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (bytes && s < d + bytes && d < s + bytes) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t groups = (n + kCopyThreads * kCopyVec - 1) / (kCopyThreads * kCopyVec);
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(groups)), dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError();
}
