// fp32 GEMMs on the matrix cores (v_mfma_f32_16x16x4_f32), for the fp32
// layer: the projection f1 with its SiLU and U/V/Q/K split, the output f2
// with bias and residual ("万亿参数推荐大模型…" §2.1 first and third
// equations), and the products of the backward pass (strided operands,
// split-K with atomic accumulation for the weight gradients).
//
//   C[m, n] = sum_k A[m sam + k sak] B[k sbk + n sbn]
//
// Each operand is taken with its k index contiguous (sak == 1, sbk == 1)
// or with its m / n index contiguous (sam == 1, sbn == 1); other layouts
// are refused and the caller uses its plain kernel. A workgroup computes a
// 128 x 128 tile with 4 waves of 64 x 64 (4 x 4 tiles of 16 x 16), staging K
// in chunks of 16 through two LDS buffers: row-major [row][k] with 4 floats
// of padding, so that a lane's float4 of k values is one conflict-free b128
// read, and the contraction step e of a chunk pairs k = 4g + e across the
// lane groups g.
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 16, kLd = kBK + 4;
constexpr float kLog2eG = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float comp4(const float4& v, int e) {
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// One operand chunk: rows [row0, row0 + 128) x k [k0, k0 + 16) of
// X[row][k] = P[row * s_row + k * s_k], two float4 of four k values per
// thread, zero outside rows < nrows and k < kend. KC: s_k == 1 (one float4
// load); else s_row == 1 (four scalar loads, each coalesced over the lanes'
// consecutive rows). Either way a thread's float4 is one conflict-free LDS
// write; transposing four-row float4s with scalar LDS writes instead put 32
// lanes on 4 banks and cost the products with such operands 4 % of the
// backward pass.
template <bool KC>
__device__ __forceinline__ void chunk_load(const float* __restrict__ P, int64_t s_row, int64_t s_k, int row0,
                                           int nrows, int64_t k0, int64_t kend, int tid, float4 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    if constexpr (KC) {
      const int row = row0 + (idx >> 2);
      const int64_t k = k0 + 4 * (idx & 3);
      if (row < nrows && k + 3 < kend) {
        r[i] = *reinterpret_cast<const float4*>(P + row * s_row + k);
      } else {
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (row < nrows && k + e < kend) ? P[row * s_row + k + e] : 0.0f;
        r[i] = make_float4(t[0], t[1], t[2], t[3]);
      }
    } else {
      // four k values of one row: each is a coalesced scalar load across the
      // lanes (consecutive rows), and the float4 goes to LDS in one write
      const int row = row0 + (idx & 127);
      const int64_t k = k0 + 4 * (idx >> 7);
      float t[4];
      if (row < nrows && k + 3 < kend) {
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = P[row + (k + e) * s_k];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (row < nrows && k + e < kend) ? P[row + (k + e) * s_k] : 0.0f;
      }
      r[i] = make_float4(t[0], t[1], t[2], t[3]);
    }
  }
}

template <bool KC>
__device__ __forceinline__ void chunk_store(float (*S)[kLd], int tid, const float4 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    if constexpr (KC) {
      *reinterpret_cast<float4*>(&S[idx >> 2][4 * (idx & 3)]) = r[i];
    } else {
      *reinterpret_cast<float4*>(&S[idx & 127][4 * (idx >> 7)]) = r[i];
    }
  }
}

// EPI: 0 store C (+ bias[n] + addend[m, n]); 1 atomic add into C; 2 SiLU of
// (acc + bias[n]) split into outs[n / split], and the pre-activation into C
// when C is set.
template <bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_mma_kernel(GemmF32Args p) {
  __shared__ __attribute__((aligned(16))) float sA[2][kBM][kLd];
  __shared__ __attribute__((aligned(16))) float sB[2][kBN][kLd];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i = l & 15, g = l >> 4;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * p.kchunk;
  const int64_t kend = min(p.K, kbeg + p.kchunk);
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{};

  float4 ra[2], rb[2];
  const int nchunks = kend > kbeg ? static_cast<int>((kend - kbeg + kBK - 1) / kBK) : 0;
  if (nchunks > 0) {
    chunk_load<A_KC>(p.A, p.sam, p.sak, m0, p.M, kbeg, kend, tid, ra);
    chunk_load<B_KC>(p.B, p.sbn, p.sbk, n0, p.N, kbeg, kend, tid, rb);
    chunk_store<A_KC>(sA[0], tid, ra);
    chunk_store<B_KC>(sB[0], tid, rb);
  }
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      const int64_t k0 = kbeg + static_cast<int64_t>(c + 1) * kBK;
      chunk_load<A_KC>(p.A, p.sam, p.sak, m0, p.M, k0, kend, tid, ra);
      chunk_load<B_KC>(p.B, p.sbn, p.sbk, n0, p.N, k0, kend, tid, rb);
    }
    float4 a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = *reinterpret_cast<const float4*>(&sA[buf][wm + 16 * t + i][4 * g]);
      b[t] = *reinterpret_cast<const float4*>(&sB[buf][wn + 16 * t + i][4 * g]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma(comp4(a[mt], e), comp4(b[nt], e), acc[mt][nt]);
    if (more) {
      chunk_store<A_KC>(sA[buf ^ 1], tid, ra);
      chunk_store<B_KC>(sB[buf ^ 1], tid, rb);
    }
    __syncthreads();
  }

  // accumulator register r of tile (mt, nt): row wm + 16 mt + 4g + r, column wn + 16 nt + i
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = n0 + wn + 16 * nt + i;
    const bool nok = n < p.N;
    const float bn = (EPI != 1 && p.bias && nok) ? p.bias[n] : 0.0f;
    float* out = nullptr;
    int col = 0;
    if constexpr (EPI == 2) {
      // the 16 columns of this tile lie in one output (split % 16 == 0)
      const int tile0 = n0 + wn + 16 * nt;
      const int o = tile0 / p.split;
      out = o == 0 ? p.outs[0] : (o == 1 ? p.outs[1] : (o == 2 ? p.outs[2] : p.outs[3]));
      col = n - o * p.split;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * mt + 4 * g + r;
        if (!nok || m >= p.M) continue;
        const float v = acc[mt][nt][r];
        if constexpr (EPI == 0) {
          float y = v + bn;
          if (p.addend) y += p.addend[static_cast<int64_t>(m) * p.ldc + n];
          p.C[static_cast<int64_t>(m) * p.ldc + n] = y;
        } else if constexpr (EPI == 1) {
          atomicAdd(&p.C[static_cast<int64_t>(m) * p.ldc + n], v);
        } else {
          const float z = v + bn;
          if (p.C) p.C[static_cast<int64_t>(m) * p.ldc + n] = z;
          out[static_cast<int64_t>(m) * p.split + col] =
              z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2eG * z));
        }
      }
  }
}

bool aligned16p(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <int EPI>
hipError_t dispatch(const GemmF32Args& a, dim3 grid, hipStream_t s) {
  const bool akc = a.sak == 1, bkc = a.sbk == 1;
  if (akc && bkc)
    hipLaunchKernelGGL((gemm_f32_mma_kernel<true, true, EPI>), grid, dim3(256), 0, s, a);
  else if (akc)
    hipLaunchKernelGGL((gemm_f32_mma_kernel<true, false, EPI>), grid, dim3(256), 0, s, a);
  else if (bkc)
    hipLaunchKernelGGL((gemm_f32_mma_kernel<false, true, EPI>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_f32_mma_kernel<false, false, EPI>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32_mma(const GemmF32Args& a, int epi, int splits, hipStream_t s) {
  // operand layouts this kernel takes: one index of each operand contiguous,
  // the other stride a multiple of 4 floats, 16-byte aligned bases
  const bool a_ok = aligned16p(a.A) && ((a.sak == 1 && a.sam % 4 == 0) || (a.sam == 1 && a.sak % 4 == 0));
  const bool b_ok = aligned16p(a.B) && ((a.sbk == 1 && a.sbn % 4 == 0) || (a.sbn == 1 && a.sbk % 4 == 0));
  if (!a_ok || !b_ok || a.M < 0 || a.N < 0 || a.K < 0) return hipErrorNotSupported;
  if (epi == 2 && (a.split <= 0 || a.split % 16 != 0 || a.N > 4 * a.split)) return hipErrorNotSupported;
  if (epi != 1 && splits != 1) return hipErrorNotSupported;
  if (a.M == 0 || a.N == 0) return hipSuccess;
  GemmF32Args p = a;
  int z = 1;
  if (splits > 1) {
    int64_t kc = (a.K + splits - 1) / splits;
    kc = (kc + kBK - 1) / kBK * kBK;
    p.kchunk = kc > 0 ? kc : kBK;
    z = static_cast<int>((a.K + p.kchunk - 1) / p.kchunk);
    if (z < 1) z = 1;
  } else {
    p.kchunk = a.K > 0 ? a.K : 1;
  }
  const int64_t gm = (static_cast<int64_t>(a.M) + kBM - 1) / kBM;
  if (gm > 65535) return hipErrorNotSupported;
  dim3 grid((a.N + kBN - 1) / kBN, static_cast<unsigned>(gm), z);
  // under 8 workgroups each K chunk's load latency is exposed: the plain
  // kernels, with many small blocks, are faster there
  if (static_cast<int64_t>(grid.x) * grid.y * grid.z < 8) return hipErrorNotSupported;
  if (epi == 0) return dispatch<0>(p, grid, s);
  if (epi == 1) return dispatch<1>(p, grid, s);
  if (!(p.sak == 1 && p.sbk == 1)) return hipErrorNotSupported;
  hipLaunchKernelGGL((gemm_f32_mma_kernel<true, true, 2>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hstu
