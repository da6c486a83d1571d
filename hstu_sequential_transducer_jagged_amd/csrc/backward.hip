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

// Zero fill of several buffers in one launch: blockIdx.y picks the buffer.
__global__ __launch_bounds__(256) void fill_zero_list_kernel(ZeroList z) {
  float* const p = z.p[blockIdx.y];
  const int64_t n = z.n[blockIdx.y];
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

// The row kernels below hold a row of d <= 1024 floats in registers, as up
// to four float4 per lane (float4 i of lane l covers columns 4 (l + 64 i) ..
// +3), read once with 16-byte loads.
constexpr int kRow4 = 4;

__device__ __forceinline__ float4 ld4(const float* p, int c4, int n4) {
  return c4 < n4 ? *reinterpret_cast<const float4*>(p + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
}
__device__ __forceinline__ float4 ld4_or(const float* p, int c4, float v) {
  return p ? *reinterpret_cast<const float4*>(p + 4 * c4) : make_float4(v, v, v, v);
}

// Per row (one wave): N^ = (AV - mean) * rstd, G = (N^ gamma + beta) . U.
// Keeps N^ and rstd for the backward. d % 4 == 0.
__global__ __launch_bounds__(256) void ln_gate_fwd_kernel(const float* __restrict__ av,
                                                          const float* __restrict__ u,
                                                          const float* gamma, const float* beta,
                                                          float* nhat, float* rstd_out, float* g,
                                                          uint16_t* g16, int64_t M, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int n4 = d >> 2;
  const float* x = av + row * d;
  float4 xv[kRow4];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kRow4; ++i) {
    xv[i] = ld4(x, lane + 64 * i, n4);
    s += (xv[i].x + xv[i].y) + (xv[i].z + xv[i].w);
  }
  const float mean = wave_sum(s) / static_cast<float>(d);
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kRow4; ++i) {
    if (lane + 64 * i >= n4) continue;
    const float a0 = xv[i].x - mean, a1 = xv[i].y - mean, a2 = xv[i].z - mean, a3 = xv[i].w - mean;
    ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < kRow4; ++i) {
    const int c4 = lane + 64 * i;
    if (c4 >= n4) continue;
    const float4 gm = ld4_or(gamma, c4, 1.0f), bt = ld4_or(beta, c4, 0.0f);
    const float4 uv = *reinterpret_cast<const float4*>(u + row * d + 4 * c4);
    const float4 n = make_float4((xv[i].x - mean) * rstd, (xv[i].y - mean) * rstd, (xv[i].z - mean) * rstd,
                                 (xv[i].w - mean) * rstd);
    *reinterpret_cast<float4*>(nhat + row * d + 4 * c4) = n;
    const float4 o = make_float4((n.x * gm.x + bt.x) * uv.x, (n.y * gm.y + bt.y) * uv.y,
                                 (n.z * gm.z + bt.z) * uv.z, (n.w * gm.w + bt.w) * uv.w);
    if (g16)
      *reinterpret_cast<uint2*>(g16 + row * d + 4 * c4) = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
    else
      *reinterpret_cast<float4*>(g + row * d + 4 * c4) = o;
  }
  if (lane == 0) rstd_out[row] = rstd;
}

// Per row (one wave), from dG: dU (into dz's U block), dAV, and this
// block's partial column sums of dN . N^ (dgamma) and dN (dbeta), dN = dG . U.
// d % 4 == 0, ldu % 4 == 0.
__global__ __launch_bounds__(256) void ln_gate_bwd_kernel(const float* __restrict__ dg,
                                                          const float* __restrict__ u,
                                                          const float* __restrict__ nhat,
                                                          const float* __restrict__ rstd,
                                                          const float* gamma, const float* beta,
                                                          float* du, int64_t ldu, float* dav,
                                                          uint16_t* dav16, float* dgamma, float* dbeta,
                                                          int64_t M, int d) {
  __shared__ __attribute__((aligned(16))) float sg[4][1024];
  __shared__ __attribute__((aligned(16))) float sb[4][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n4 = d >> 2;
  float4 gsum[kRow4], bsum[kRow4];
#pragma unroll
  for (int i = 0; i < kRow4; ++i) gsum[i] = bsum[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + wave; row < M &&
       row < static_cast<int64_t>(blockIdx.x) * 16 + 16; row += 4) {
    float4 dnh[kRow4], nh[kRow4];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < kRow4; ++i) {
      const int c4 = lane + 64 * i;
      if (c4 >= n4) {
        dnh[i] = nh[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        continue;
      }
      const int64_t o = row * d + 4 * c4;
      const float4 gm = ld4_or(gamma, c4, 1.0f), bt = ld4_or(beta, c4, 0.0f);
      const float4 g4 = *reinterpret_cast<const float4*>(dg + o);
      const float4 u4 = *reinterpret_cast<const float4*>(u + o);
      nh[i] = *reinterpret_cast<const float4*>(nhat + o);
      *reinterpret_cast<float4*>(du + row * ldu + 4 * c4) =
          make_float4(g4.x * (nh[i].x * gm.x + bt.x), g4.y * (nh[i].y * gm.y + bt.y),
                      g4.z * (nh[i].z * gm.z + bt.z), g4.w * (nh[i].w * gm.w + bt.w));
      const float4 dn = make_float4(g4.x * u4.x, g4.y * u4.y, g4.z * u4.z, g4.w * u4.w);
      gsum[i].x += dn.x * nh[i].x; gsum[i].y += dn.y * nh[i].y;
      gsum[i].z += dn.z * nh[i].z; gsum[i].w += dn.w * nh[i].w;
      bsum[i].x += dn.x; bsum[i].y += dn.y; bsum[i].z += dn.z; bsum[i].w += dn.w;
      dnh[i] = make_float4(dn.x * gm.x, dn.y * gm.y, dn.z * gm.z, dn.w * gm.w);
      s1 += (dnh[i].x + dnh[i].y) + (dnh[i].z + dnh[i].w);
      s2 += (dnh[i].x * nh[i].x + dnh[i].y * nh[i].y) + (dnh[i].z * nh[i].z + dnh[i].w * nh[i].w);
    }
    const float m1 = wave_sum(s1) / static_cast<float>(d);
    const float m2 = wave_sum(s2) / static_cast<float>(d);
    const float r = rstd[row];
#pragma unroll
    for (int i = 0; i < kRow4; ++i) {
      const int c4 = lane + 64 * i;
      if (c4 >= n4) continue;
      const float4 o = make_float4(r * (dnh[i].x - m1 - nh[i].x * m2), r * (dnh[i].y - m1 - nh[i].y * m2),
                                   r * (dnh[i].z - m1 - nh[i].z * m2), r * (dnh[i].w - m1 - nh[i].w * m2));
      if (dav16)
        *reinterpret_cast<uint2*>(dav16 + row * d + 4 * c4) = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      else
        *reinterpret_cast<float4*>(dav + row * d + 4 * c4) = o;
    }
  }
#pragma unroll
  for (int i = 0; i < kRow4; ++i) {
    const int c4 = lane + 64 * i;
    if (c4 < n4) {
      *reinterpret_cast<float4*>(&sg[wave][4 * c4]) = gsum[i];
      *reinterpret_cast<float4*>(&sb[wave][4 * c4]) = bsum[i];
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

// dZ = d[U V Q K] . SiLU'(Z) for the bf16 products, in 64 x 64 tiles: dZ in
// bf16 row-major (dz16 [T, n], the A operand of dX = dZ W1), dZ^T in bf16
// with tp columns, zero past T (dzt [n, tp], the A operand of
// dW1 = dZ^T Xin), and the column sums of dZ in fp32 added to db1 (one
// atomic per column and tile). The fp32 dZ is not written back.
__global__ __launch_bounds__(256) void silu_bwd_bf16_kernel(const float* __restrict__ dz,
                                                            const float* __restrict__ z, int64_t T, int n,
                                                            uint16_t* __restrict__ dz16,
                                                            uint16_t* __restrict__ dzt, int64_t tp,
                                                            float* db1) {
  __shared__ float t[64][65];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * 16 + (tid >> 4);
    const int c = (tid & 15) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + r < T && c0 + c < n) {
      const int64_t o = (r0 + r) * n + c0 + c;
      const float4 g = *reinterpret_cast<const float4*>(dz + o);
      const float4 zz = *reinterpret_cast<const float4*>(z + o);
      float sg;
      sg = sigmoid_f(zz.x); v.x = g.x * sg * (1.0f + zz.x * (1.0f - sg));
      sg = sigmoid_f(zz.y); v.y = g.y * sg * (1.0f + zz.y * (1.0f - sg));
      sg = sigmoid_f(zz.z); v.z = g.z * sg * (1.0f + zz.z * (1.0f - sg));
      sg = sigmoid_f(zz.w); v.w = g.w * sg * (1.0f + zz.w * (1.0f - sg));
      *reinterpret_cast<uint2*>(dz16 + o) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
    t[r][c + 0] = v.x;
    t[r][c + 1] = v.y;
    t[r][c + 2] = v.z;
    t[r][c + 3] = v.w;
  }
  __syncthreads();
  if (tid < 64 && c0 + tid < n && r0 < T) {
    float sum = 0.0f;
    for (int r = 0; r < 64; ++r) sum += t[r][tid];
    atomicAdd(&db1[c0 + tid], sum);
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = it * 256 + tid;
    const int cc = idx >> 3;
    const int ch = idx & 7;
    if (c0 + cc < n && r0 + ch * 8 < tp) {
      uint4 o;
      o.x = pack_bf16x2(t[ch * 8 + 0][cc], t[ch * 8 + 1][cc]);
      o.y = pack_bf16x2(t[ch * 8 + 2][cc], t[ch * 8 + 3][cc]);
      o.z = pack_bf16x2(t[ch * 8 + 4][cc], t[ch * 8 + 5][cc]);
      o.w = pack_bf16x2(t[ch * 8 + 6][cc], t[ch * 8 + 7][cc]);
      *reinterpret_cast<uint4*>(dzt + static_cast<int64_t>(c0 + cc) * tp + r0 + ch * 8) = o;
    }
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

hipError_t launch_fill_zero_list(const ZeroList& z, hipStream_t s) {
  if (z.count < 0 || z.count > kZeroListMax) return hipErrorInvalidValue;
  int64_t most = 0;
  for (int i = 0; i < z.count; ++i) {
    if (z.n[i] < 0 || (z.n[i] > 0 && z.p[i] == nullptr)) return hipErrorInvalidValue;
    most = z.n[i] > most ? z.n[i] : most;
  }
  if (most == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_list_kernel, dim3(blocks_for(most), static_cast<unsigned>(z.count)), dim3(256), 0,
                     s, z);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* X, int64_t ldx, int64_t M, int N, float* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((N + 255) / 256, static_cast<unsigned>((M + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(colsum_kernel, grid, dim3(256), 0, s, X, ldx, M, N, out);
  return hipGetLastError();
}

hipError_t launch_ln_gate_fwd(const float* av, const float* u, const float* gamma, const float* beta,
                              float* nhat, float* rstd, float* g, uint16_t* g16, int64_t M, int d, float eps,
                              hipStream_t s) {
  if (M == 0) return hipSuccess;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (d % 4 != 0 || d > 64 * 4 * kRow4 || !a16(av) || !a16(u) || !a16(nhat) || !a16(g) || !a16(gamma) ||
      !a16(beta) || (reinterpret_cast<uintptr_t>(g16) & 7u) != 0 || (g == nullptr && g16 == nullptr))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ln_gate_fwd_kernel, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, s, av, u,
                     gamma, beta, nhat, rstd, g, g16, M, d, eps);
  return hipGetLastError();
}

hipError_t launch_ln_gate_bwd(const float* dg, const float* u, const float* nhat, const float* rstd,
                              const float* gamma, const float* beta, float* du, int64_t ldu, float* dav,
                              uint16_t* dav16, float* dgamma, float* dbeta, int64_t M, int d, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (d % 4 != 0 || d > 64 * 4 * kRow4 || ldu % 4 != 0 || !a16(dg) || !a16(u) || !a16(nhat) || !a16(du) ||
      !a16(dav) || !a16(gamma) || !a16(beta) || (reinterpret_cast<uintptr_t>(dav16) & 7u) != 0 ||
      (dav == nullptr && dav16 == nullptr))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ln_gate_bwd_kernel, dim3(static_cast<unsigned>((M + 15) / 16)), dim3(256), 0, s, dg,
                     u, nhat, rstd, gamma, beta, du, ldu, dav, dav16, dgamma, dbeta, M, d);
  return hipGetLastError();
}

hipError_t launch_silu_bwd(float* dz, const float* z, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_bwd_kernel, dim3(blocks_for(n)), dim3(256), 0, s, dz, z, n);
  return hipGetLastError();
}

hipError_t launch_silu_bwd_bf16(const float* dz, const float* z, int64_t T, int n, uint16_t* dz16,
                                uint16_t* dzt, int64_t tp, float* db1, hipStream_t s) {
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (n % 4 != 0 || tp % 8 != 0 || tp < T || !a16(dz) || !a16(z) || !a16(dz16) || !a16(dzt)) return hipErrorInvalidValue;
  if (n == 0 || tp == 0) return hipSuccess;
  const int64_t gx = (tp + 63) / 64;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(silu_bwd_bf16_kernel, dim3(static_cast<unsigned>(gx), (n + 63) / 64), dim3(256), 0, s, dz,
                     z, T, n, dz16, dzt, tp, db1);
  return hipGetLastError();
}


}  // namespace hstu
