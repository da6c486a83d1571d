// f1 and f2 of the HSTU layer on gfx950 MFMA ("万亿参数推荐大模型：HSTU 架构
// 如何超越传统 Self-Attention" §2.1: f1 and f2 are single linear layers).
//
//   proj: [U|V|Q|K] = SiLU(X W1^T + b1), the SiLU and the four-way split are
//         the epilogue (first equation of §2.1);
//   out:  Y = X + G W2^T + b2, bias and residual are the epilogue (third
//         equation plus the block diagram's skip connection).
//
// Both are C[M, N] = A[M, K] B[N, K]^T with A and B row-major and K
// contiguous, which is exactly the operand layout of
// v_mfma_f32_16x16x32_bf16 (lane = row, 8 consecutive k), so tiles are
// staged through LDS unchanged. Block tile 128 x 128, K step 32, four waves
// of 64 x 64; the next K step's global loads are issued before the current
// step's MFMAs.
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

constexpr int kTM = 128;
constexpr int kTN = 128;
constexpr int kTK = 32;
constexpr int kLdsRow = kTK + 8;   // bf16 per LDS row (+16 B pad)

__device__ __forceinline__ float silu_exact(float z) { return z / (1.0f + __expf(-z)); }

struct ProjEpi {
  const float* bias;
  uint16_t* out[4];
  int K;
  __device__ __forceinline__ void operator()(int64_t m, int n, float acc) const {
    const float z = acc + (bias ? bias[n] : 0.0f);
    const int chunk = n / K;
    const int c = n - chunk * K;
    out[chunk][m * K + c] = f2bf(silu_exact(z));
  }
};

struct OutEpi {
  const float* bias;
  const uint16_t* x;
  uint16_t* y;
  int K;
  __device__ __forceinline__ void operator()(int64_t m, int n, float acc) const {
    const float r = acc + (bias ? bias[n] : 0.0f) + bf2f(x[m * K + n]);
    y[m * K + n] = f2bf(r);
  }
};

template <class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        int64_t M, int N, int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kTM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kTN * kLdsRow];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kTM;
  const int n0 = blockIdx.y * kTN;

  // each thread stages two 16-byte chunks of A and two of B per K step
  // chunk c in [0, 512): row c/4, k offset (c%4)*8
  uint4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 2;
      const int kc = (c & 3) * 8;
      const int64_t am = m0 + r;
      ra[i] = am < M ? *reinterpret_cast<const uint4*>(A + am * K + k0 + kc) : make_uint4(0, 0, 0, 0);
      const int bn = n0 + r;
      rb[i] = bn < N ? *reinterpret_cast<const uint4*>(B + static_cast<int64_t>(bn) * K + k0 + kc)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 2;
      const int kc = (c & 3) * 8;
      *reinterpret_cast<uint4*>(&sA[r * kLdsRow + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&sB[r * kLdsRow + kc]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int k0 = 0; k0 < K; k0 += kTK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + kTK < K) load(k0 + kTK);
    bf16x8 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(&sA[(wm * 64 + i * 16 + l16) * kLdsRow + 8 * g]));
      bfr[i] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(&sB[(wn * 64 + i * 16 + l16) * kLdsRow + 8 * g]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
  }

  // C layout: lane holds rows 4g + r, column lane%16 of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + l16;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + i * 16 + 4 * g + r;
        if (m < M) epi(m, n, acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// fp32: 16 x 16 output tile per block, K staged through LDS in steps of 16.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B, int64_t M,
                                                       int N, int K, Epi epi) {
  __shared__ float sA[16][17];
  __shared__ float sB[16][17];
  const int tx = threadIdx.x & 15;
  const int ty = threadIdx.x >> 4;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 16 + ty;
  const int n = blockIdx.y * 16 + tx;
  float acc = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int64_t am = static_cast<int64_t>(blockIdx.x) * 16 + ty;
    const int bn = blockIdx.y * 16 + ty;
    sA[ty][tx] = (am < M && k0 + tx < K) ? A[am * K + k0 + tx] : 0.0f;
    sB[ty][tx] = (bn < N && k0 + tx < K) ? B[static_cast<int64_t>(bn) * K + k0 + tx] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sA[ty][kk], sB[tx][kk], acc);
    __syncthreads();
  }
  if (m < M && n < N) epi(m, n, acc);
}

struct ProjEpiF32 {
  const float* bias;
  float* out[4];
  int K;
  __device__ __forceinline__ void operator()(int64_t m, int n, float acc) const {
    const float z = acc + (bias ? bias[n] : 0.0f);
    const int chunk = n / K;
    out[chunk][m * K + (n - chunk * K)] = z / (1.0f + expf(-z));
  }
};

struct OutEpiF32 {
  const float* bias;
  const float* x;
  float* y;
  int K;
  __device__ __forceinline__ void operator()(int64_t m, int n, float acc) const {
    y[m * K + n] = acc + (bias ? bias[n] : 0.0f) + x[m * K + n];
  }
};

}  // namespace

hipError_t launch_proj_bf16(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const int N = 4 * a.K;
  ProjEpi epi{a.bias,
              {static_cast<uint16_t*>(a.out[0]), static_cast<uint16_t*>(a.out[1]),
               static_cast<uint16_t*>(a.out[2]), static_cast<uint16_t*>(a.out[3])},
              a.K};
  dim3 grid(static_cast<unsigned>((a.M + kTM - 1) / kTM), (N + kTN - 1) / kTN);
  hipLaunchKernelGGL(gemm_bf16_kernel<ProjEpi>, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.w), a.M,
                     N, a.K, epi);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  OutEpi epi{a.bias, static_cast<const uint16_t*>(a.x), static_cast<uint16_t*>(a.y), a.K};
  dim3 grid(static_cast<unsigned>((a.M + kTM - 1) / kTM), (a.K + kTN - 1) / kTN);
  hipLaunchKernelGGL(gemm_bf16_kernel<OutEpi>, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.g), static_cast<const uint16_t*>(a.w), a.M,
                     a.K, a.K, epi);
  return hipGetLastError();
}

hipError_t launch_proj_f32(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const int N = 4 * a.K;
  ProjEpiF32 epi{a.bias,
                 {static_cast<float*>(a.out[0]), static_cast<float*>(a.out[1]),
                  static_cast<float*>(a.out[2]), static_cast<float*>(a.out[3])},
                 a.K};
  dim3 grid(static_cast<unsigned>((a.M + 15) / 16), (N + 15) / 16);
  hipLaunchKernelGGL(gemm_f32_kernel<ProjEpiF32>, grid, dim3(256), 0, s,
                     static_cast<const float*>(a.x), static_cast<const float*>(a.w), a.M, N,
                     a.K, epi);
  return hipGetLastError();
}

hipError_t launch_out_f32(const OutArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  OutEpiF32 epi{a.bias, static_cast<const float*>(a.x), static_cast<float*>(a.y), a.K};
  dim3 grid(static_cast<unsigned>((a.M + 15) / 16), (a.K + 15) / 16);
  hipLaunchKernelGGL(gemm_f32_kernel<OutEpiF32>, grid, dim3(256), 0, s,
                     static_cast<const float*>(a.g), static_cast<const float*>(a.w), a.M, a.K,
                     a.K, epi);
  return hipGetLastError();
}

}  // namespace hstu
