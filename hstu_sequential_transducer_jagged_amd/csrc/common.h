// Device helpers shared by the gfx950 kernels: bf16 storage conversion and
// the MFMA operand vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (one v_cvt_pk_bf16_f32), lo in bits 0..15
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum over the 64 lanes of a wave (butterfly; every lane gets the sum).
// min(nb - 1, floor(log2(|dt| + 1))) in integers (the rab time bucket).
__device__ __forceinline__ int time_bucket64(int64_t dt, int nb) {
  uint64_t a = dt < 0 ? (0ull - static_cast<uint64_t>(dt)) : static_cast<uint64_t>(dt);
  a += 1ull;
  const int b = 63 - __clzll(static_cast<long long>(a));
  return b < nb - 1 ? b : nb - 1;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

constexpr int kNgMaxChunks = 4;   // float4 chunks per lane: d <= 1024

// Token rows of G = (LayerNorm_d(av) * gamma + beta) (.) u, NR rows at a
// time, computed by one wave: lane owns the float4 chunks lane + 64 i of each
// row; mean and biased variance are two register passes reduced by
// wave_sum. The NR rows go through each step together, so the latencies of
// their cross-lane reductions overlap; each row's arithmetic is the same for
// any NR. The rows of av may sit in global memory or in LDS: the norm_gate
// kernel and the fused attention epilogue share this code and so give
// bitwise the same G. ur[r][i] holds the 4 bf16 of U for chunk lane + 64 i of
// row r, loaded by the caller (who can issue those loads early); rows with
// g[r] == nullptr are skipped.
template <int NR>
__device__ __forceinline__ void norm_gate_rows_bf16(const float* const (&avr)[NR],
                                                    const uint2 (&ur)[NR][kNgMaxChunks],
                                                    uint16_t* const (&g)[NR], int d, float eps,
                                                    const float* gamma, const float* beta, int lane) {
  const int nchunk = d >> 2;
  float4 x[NR][kNgMaxChunks];
  float s[NR], mean[NR], ss[NR], rstd[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    s[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < kNgMaxChunks; ++i) {
      const int c = lane + 64 * i;
      x[r][i] = c < nchunk ? reinterpret_cast<const float4*>(avr[r])[c] : make_float4(0, 0, 0, 0);
      s[r] += (x[r][i].x + x[r][i].y) + (x[r][i].z + x[r][i].w);
    }
  }
  const float inv_d = 1.0f / static_cast<float>(d);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] += __shfl_xor(s[r], off, 64);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    mean[r] = s[r] * inv_d;
    ss[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < kNgMaxChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunk) {
        const float a0 = x[r][i].x - mean[r], a1 = x[r][i].y - mean[r];
        const float a2 = x[r][i].z - mean[r], a3 = x[r][i].w - mean[r];
        ss[r] += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int r = 0; r < NR; ++r) ss[r] += __shfl_xor(ss[r], off, 64);
#pragma unroll
  for (int r = 0; r < NR; ++r) rstd[r] = 1.0f / sqrtf(ss[r] * inv_d + eps);
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c >= nchunk) continue;
    const int col = c * 4;
    float gm[4] = {1.f, 1.f, 1.f, 1.f}, bt[4] = {0.f, 0.f, 0.f, 0.f};
    if (gamma) {
      const float4 t = *reinterpret_cast<const float4*>(gamma + col);
      gm[0] = t.x; gm[1] = t.y; gm[2] = t.z; gm[3] = t.w;
    }
    if (beta) {
      const float4 t = *reinterpret_cast<const float4*>(beta + col);
      bt[0] = t.x; bt[1] = t.y; bt[2] = t.z; bt[3] = t.w;
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (g[r] == nullptr) continue;
      const float xv[4] = {x[r][i].x, x[r][i].y, x[r][i].z, x[r][i].w};
      float n[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) n[e] = (xv[e] - mean[r]) * rstd[r] * gm[e] + bt[e];
      const float u0 = bf2f(ur[r][i].x & 0xffff), u1 = bf2f(ur[r][i].x >> 16);
      const float u2 = bf2f(ur[r][i].y & 0xffff), u3 = bf2f(ur[r][i].y >> 16);
      uint2 o;
      o.x = pack_bf16x2(n[0] * u0, n[1] * u1);
      o.y = pack_bf16x2(n[2] * u2, n[3] * u3);
      *reinterpret_cast<uint2*>(g[r] + col) = o;
    }
  }
}

// The lane's U chunks of one bf16 row (zero past the row).
__device__ __forceinline__ void load_u_chunks_bf16(const uint16_t* u_row, int d, int lane,
                                                   uint2 (&ur)[kNgMaxChunks]) {
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    ur[i] = c < (d >> 2) ? *reinterpret_cast<const uint2*>(u_row + c * 4) : make_uint2(0, 0);
  }
}

// fp32 rows: the same arithmetic with fp32 U and G.
__device__ __forceinline__ void norm_gate_row_f32(const float* avr, const float* u_row, float* g_row, int d,
                                                  float eps, const float* gamma, const float* beta, int lane) {
  const int nchunk = d >> 2;
  float4 x[kNgMaxChunks];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    x[i] = c < nchunk ? reinterpret_cast<const float4*>(avr)[c] : make_float4(0, 0, 0, 0);
    s += (x[i].x + x[i].y) + (x[i].z + x[i].w);
  }
  const float inv_d = 1.0f / static_cast<float>(d);
  const float mean = wave_sum(s) * inv_d;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunk) {
      const float a0 = x[i].x - mean, a1 = x[i].y - mean, a2 = x[i].z - mean, a3 = x[i].w - mean;
      ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float var = wave_sum(ss) * inv_d;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c >= nchunk) continue;
    const int col = c * 4;
    float gm[4] = {1.f, 1.f, 1.f, 1.f}, bt[4] = {0.f, 0.f, 0.f, 0.f};
    if (gamma) {
      const float4 t = *reinterpret_cast<const float4*>(gamma + col);
      gm[0] = t.x; gm[1] = t.y; gm[2] = t.z; gm[3] = t.w;
    }
    if (beta) {
      const float4 t = *reinterpret_cast<const float4*>(beta + col);
      bt[0] = t.x; bt[1] = t.y; bt[2] = t.z; bt[3] = t.w;
    }
    const float xv[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
    const float4 ur = *reinterpret_cast<const float4*>(u_row + col);
    const float uv[4] = {ur.x, ur.y, ur.z, ur.w};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = ((xv[e] - mean) * rstd * gm[e] + bt[e]) * uv[e];
    *reinterpret_cast<float4*>(g_row + col) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace hstu
