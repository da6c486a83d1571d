// Backward pass of one HSTU layer for generative training (plain causal
// attention over the call's own tokens: no targets, no cache), fp32.
// "HSTU：Scaling Law 的首次探索" §7.1.5 trains on whole user sequences with a
// causal forward; the gradients follow the layer's three equations
// ("万亿参数推荐大模型…" §2.1) backwards:
//
//   Y = X + G W2^T + b2          dG = dY W2, dW2 = dY^T G, db2 = sum dY
//   G = (N^ gamma + beta) . U     dU = dG . (N^ gamma + beta), dgamma, dbeta,
//                                 dAV = LayerNorm backward of dG . U . gamma
//   AV_h = (SiLU(S_h) . M) V_h    dV, dS = (dAV V^T) . SiLU'(S) . M
//   S_h = a Q_h K_h^T + rab       dQ = a dS K, dK = a dS^T Q, d tables += dS
//   [U V Q K] = SiLU(X W1^T + b1) dZ = d[U V Q K] . SiLU'(Z), dW1, db1, dX
//
// Kernels here are plain fp32: a strided tiled GEMM (split-K with atomics
// for the weight gradients) and row kernels for the LayerNorm/gate step.
// The attention backward is in attn_train.hip.
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// C[m, n] = sum_k A[m sam + k sak] B[k sbk + n sbn] over the block's K chunk
// (+ bias[n] + addend[m, n] when not split). 64 x 64 tile, 256 threads, 4 x 4
// outputs per thread, K staged 16 at a time. ATOMIC: the chunk's sum is added
// to C (C zeroed beforehand; no bias or addend).
template <bool ATOMIC>
__global__ __launch_bounds__(256) void gemm_f32s_kernel(const float* __restrict__ A, int64_t sam,
                                                        int64_t sak, const float* __restrict__ B,
                                                        int64_t sbk, int64_t sbn, float* C, int64_t ldc,
                                                        const float* addend, const float* bias, int M,
                                                        int N, int64_t K, int64_t kchunk) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int64_t kb = static_cast<int64_t>(blockIdx.z) * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  const bool a_kfast = sak == 1;   // which index runs along memory, for coalescing
  const bool b_nfast = sbn == 1;
  for (int64_t k0 = kb; k0 < ke; k0 += 16) {
    for (int e = tid; e < 1024; e += 256) {
      const int kk = a_kfast ? (e & 15) : (e >> 6);
      const int mm = a_kfast ? (e >> 4) : (e & 63);
      const int64_t k = k0 + kk;
      const int m = m0 + mm;
      As[kk][mm] = (m < M && k < ke) ? A[m * sam + k * sak] : 0.0f;
      const int kb2 = b_nfast ? (e >> 6) : (e & 15);
      const int nn = b_nfast ? (e & 63) : (e >> 4);
      const int64_t k2 = k0 + kb2;
      const int n = n0 + nn;
      Bs[kb2][nn] = (n < N && k2 < ke) ? B[k2 * sbk + n * sbn] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      if (ATOMIC) {
        atomicAdd(&C[m * ldc + n], acc[i][j]);
      } else {
        float v = acc[i][j];
        if (bias) v += bias[n];
        if (addend) v += addend[m * ldc + n];
        C[m * ldc + n] = v;
      }
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

// Column sums of X [M, N] (row stride ldx) added to out[N]: each block sums
// kRowsPerBlock rows per column, then one atomic per column.
constexpr int kRowsPerBlock = 64;

__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ X, int64_t ldx, int64_t M,
                                                     int N, float* out) {
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kRowsPerBlock;
  const int64_t r1 = r0 + kRowsPerBlock < M ? r0 + kRowsPerBlock : M;
  for (int n = blockIdx.x * 256 + threadIdx.x; n < N; n += gridDim.x * 256) {
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r) s += X[r * ldx + n];
    atomicAdd(&out[n], s);
  }
}

// Per row (one wave): N^ = (AV - mean) * rstd, G = (N^ gamma + beta) . U.
// Keeps N^ and rstd for the backward.
__global__ __launch_bounds__(256) void ln_gate_fwd_kernel(const float* __restrict__ av,
                                                          const float* __restrict__ u,
                                                          const float* gamma, const float* beta,
                                                          float* nhat, float* rstd_out, float* g,
                                                          int64_t M, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* x = av + row * d;
  float s = 0.0f;
  for (int c = lane; c < d; c += 64) s += x[c];
  const float mean = wave_sum(s) / static_cast<float>(d);
  float ss = 0.0f;
  for (int c = lane; c < d; c += 64) {
    const float t = x[c] - mean;
    ss += t * t;
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(d) + eps);
  for (int c = lane; c < d; c += 64) {
    const float n = (x[c] - mean) * rstd;
    nhat[row * d + c] = n;
    const float gm = gamma ? gamma[c] : 1.0f, bt = beta ? beta[c] : 0.0f;
    g[row * d + c] = (n * gm + bt) * u[row * d + c];
  }
  if (lane == 0) rstd_out[row] = rstd;
}

// Per row (one wave), from dG: dU (into dz's U block), dAV, and this
// block's partial column sums of dN . N^ (dgamma) and dN (dbeta), dN = dG . U.
__global__ __launch_bounds__(256) void ln_gate_bwd_kernel(const float* __restrict__ dg,
                                                          const float* __restrict__ u,
                                                          const float* __restrict__ nhat,
                                                          const float* __restrict__ rstd,
                                                          const float* gamma, const float* beta,
                                                          float* du, int64_t ldu, float* dav,
                                                          float* dgamma, float* dbeta, int64_t M,
                                                          int d) {
  __shared__ float sg[4][1024];
  __shared__ float sb[4][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int c = lane; c < d; c += 64) {
    sg[wave][c] = 0.0f;
    sb[wave][c] = 0.0f;
  }
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + wave; row < M &&
       row < static_cast<int64_t>(blockIdx.x) * 16 + 16; row += 4) {
    float s1 = 0.0f, s2 = 0.0f;
    for (int c = lane; c < d; c += 64) {
      const int64_t i = row * d + c;
      const float gm = gamma ? gamma[c] : 1.0f, bt = beta ? beta[c] : 0.0f;
      const float nh = nhat[i];
      du[row * ldu + c] = dg[i] * (nh * gm + bt);
      const float dn = dg[i] * u[i];
      sg[wave][c] += dn * nh;
      sb[wave][c] += dn;
      const float dnh = dn * gm;
      s1 += dnh;
      s2 += dnh * nh;
    }
    const float m1 = wave_sum(s1) / static_cast<float>(d);
    const float m2 = wave_sum(s2) / static_cast<float>(d);
    const float r = rstd[row];
    for (int c = lane; c < d; c += 64) {
      const int64_t i = row * d + c;
      const float gm = gamma ? gamma[c] : 1.0f;
      const float dnh = dg[i] * u[i] * gm;
      dav[i] = r * (dnh - m1 - nhat[i] * m2);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256) {
    atomicAdd(&dgamma[c], (sg[0][c] + sg[1][c]) + (sg[2][c] + sg[3][c]));
    atomicAdd(&dbeta[c], (sb[0][c] + sb[1][c]) + (sb[2][c] + sb[3][c]));
  }
}

// Input LayerNorm backward, per row (one wave): xhat = (x - mean) / sigma
// recomputed from x; dxh = dxn . gamma;
// dx = dy + (dxh - mean(dxh) - xhat mean(dxh . xhat)) / sigma; this block's
// partial column sums of dxn . xhat (dgamma) and dxn (dbeta).
__global__ __launch_bounds__(256) void ln1_bwd_kernel(const float* __restrict__ x, const float* __restrict__ dxn,
                                                      const float* __restrict__ dy, const float* gamma,
                                                      float* dx, float* dgamma, float* dbeta, int64_t M, int d,
                                                      float eps) {
  __shared__ float sg[4][1024];
  __shared__ float sb[4][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int c = lane; c < d; c += 64) {
    sg[wave][c] = 0.0f;
    sb[wave][c] = 0.0f;
  }
  const float inv_d = 1.0f / static_cast<float>(d);
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + wave; row < M &&
       row < static_cast<int64_t>(blockIdx.x) * 16 + 16; row += 4) {
    const float* xr = x + row * d;
    const float* gr = dxn + row * d;
    float sx = 0.0f;
    for (int c = lane; c < d; c += 64) sx += xr[c];
    const float mean = wave_sum(sx) * inv_d;
    float sv = 0.0f;
    for (int c = lane; c < d; c += 64) {
      const float t = xr[c] - mean;
      sv += t * t;
    }
    const float rstd = 1.0f / sqrtf(wave_sum(sv) * inv_d + eps);
    float s1 = 0.0f, s2 = 0.0f;
    for (int c = lane; c < d; c += 64) {
      const float xh = (xr[c] - mean) * rstd;
      const float g = gr[c];
      sg[wave][c] += g * xh;
      sb[wave][c] += g;
      const float dxh = g * (gamma ? gamma[c] : 1.0f);
      s1 += dxh;
      s2 += dxh * xh;
    }
    const float m1 = wave_sum(s1) * inv_d;
    const float m2 = wave_sum(s2) * inv_d;
    for (int c = lane; c < d; c += 64) {
      const float xh = (xr[c] - mean) * rstd;
      const float dxh = gr[c] * (gamma ? gamma[c] : 1.0f);
      dx[row * d + c] = dy[row * d + c] + rstd * (dxh - m1 - xh * m2);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256) {
    atomicAdd(&dgamma[c], (sg[0][c] + sg[1][c]) + (sg[2][c] + sg[3][c]));
    atomicAdd(&dbeta[c], (sb[0][c] + sb[1][c]) + (sb[2][c] + sb[3][c]));
  }
}

// dz *= SiLU'(z), elementwise over [M, n4].
__global__ __launch_bounds__(256) void silu_bwd_kernel(float* dz, const float* __restrict__ z, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const float zz = z[i];
    const float s = sigmoid_f(zz);
    dz[i] *= s * (1.0f + zz * (1.0f - s));
  }
}

int blocks_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<int>(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

hipError_t launch_gemm_f32s(const float* A, int64_t sam, int64_t sak, const float* B, int64_t sbk,
                            int64_t sbn, float* C, int64_t ldc, const float* addend, const float* bias,
                            int M, int N, int64_t K, int splits, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  {
    GemmF32Args g{};
    g.A = A; g.sam = sam; g.sak = sak;
    g.B = B; g.sbk = sbk; g.sbn = sbn;
    g.C = C; g.ldc = ldc;
    g.M = M; g.N = N; g.K = K;
    if (splits > 1) {
      const hipError_t e = launch_gemm_f32_mma(g, 1, splits, s);
      if (e != hipErrorNotSupported) return e;
    } else {
      g.addend = addend; g.bias = bias;
      const hipError_t e = launch_gemm_f32_mma(g, 0, 1, s);
      if (e != hipErrorNotSupported) return e;
    }
  }
  if (splits > 1) {
    int64_t kchunk = (K + splits - 1) / splits;
    kchunk = (kchunk + 15) / 16 * 16;
    const int z = static_cast<int>((K + kchunk - 1) / kchunk);
    dim3 grid((N + 63) / 64, (M + 63) / 64, z > 0 ? z : 1);
    hipLaunchKernelGGL(gemm_f32s_kernel<true>, grid, dim3(256), 0, s, A, sam, sak, B, sbk, sbn, C, ldc,
                       nullptr, nullptr, M, N, K, kchunk);
  } else {
    dim3 grid((N + 63) / 64, (M + 63) / 64, 1);
    hipLaunchKernelGGL(gemm_f32s_kernel<false>, grid, dim3(256), 0, s, A, sam, sak, B, sbk, sbn, C, ldc,
                       addend, bias, M, N, K, K);
  }
  return hipGetLastError();
}

hipError_t launch_ln1_bwd(const float* x, const float* dxn, const float* dy, const float* gamma, float* dx,
                          float* dgamma, float* dbeta, int64_t M, int d, float eps, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(ln1_bwd_kernel, dim3(static_cast<unsigned>((M + 15) / 16)), dim3(256), 0, s, x, dxn, dy,
                     gamma, dx, dgamma, dbeta, M, d, eps);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* X, int64_t ldx, int64_t M, int N, float* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((N + 255) / 256, static_cast<unsigned>((M + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(colsum_kernel, grid, dim3(256), 0, s, X, ldx, M, N, out);
  return hipGetLastError();
}

hipError_t launch_ln_gate_fwd(const float* av, const float* u, const float* gamma, const float* beta,
                              float* nhat, float* rstd, float* g, int64_t M, int d, float eps,
                              hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(ln_gate_fwd_kernel, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, s, av, u,
                     gamma, beta, nhat, rstd, g, M, d, eps);
  return hipGetLastError();
}

hipError_t launch_ln_gate_bwd(const float* dg, const float* u, const float* nhat, const float* rstd,
                              const float* gamma, const float* beta, float* du, int64_t ldu, float* dav,
                              float* dgamma, float* dbeta, int64_t M, int d, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(ln_gate_bwd_kernel, dim3(static_cast<unsigned>((M + 15) / 16)), dim3(256), 0, s, dg,
                     u, nhat, rstd, gamma, beta, du, ldu, dav, dgamma, dbeta, M, d);
  return hipGetLastError();
}

hipError_t launch_silu_bwd(float* dz, const float* z, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_bwd_kernel, dim3(blocks_for(n)), dim3(256), 0, s, dz, z, n);
  return hipGetLastError();
}


}  // namespace hstu
