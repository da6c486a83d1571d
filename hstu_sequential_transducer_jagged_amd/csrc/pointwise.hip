// Bandwidth-bound pointwise kernels for gfx950.
//
// norm_gate: G = (LayerNorm_d(AV) * gamma + beta) (.) U, the first half of
//   the pointwise transformation ("万亿参数推荐大模型：HSTU 架构如何超越传统
//   Self-Attention" §2.1, third equation and block diagram: LayerNorm, then
//   the product with U). One wavefront per token row; each lane owns float4
//   chunks spaced 64 chunks apart so every load and store is a coalesced
//   16-byte (AV) or 8-byte (bf16 U/G) access; mean and variance are two
//   register passes reduced with cross-lane shuffles (no LDS round trip).
//
// embed: X[t] = item_emb[id_t] + action_emb[a_t], the action-oriented token
//   of "6.2. HSTU的工程突破" eq. 6.2.2. One wavefront per token, 16-byte
//   gathers of the two rows, fp32 add, one rounding.
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

constexpr int kMaxChunks = 4;   // float4 chunks per lane: d <= 1024

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int d = a.d;
  const int nchunk = d >> 2;
  const float* avr = a.av + row * d;
  float4 x[kMaxChunks];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    x[i] = c < nchunk ? reinterpret_cast<const float4*>(avr)[c] : make_float4(0, 0, 0, 0);
    s += (x[i].x + x[i].y) + (x[i].z + x[i].w);
  }
  const float inv_d = 1.0f / static_cast<float>(d);
  const float mean = wave_sum(s) * inv_d;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunk) {
      const float a0 = x[i].x - mean, a1 = x[i].y - mean, a2 = x[i].z - mean, a3 = x[i].w - mean;
      ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float var = wave_sum(ss) * inv_d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c >= nchunk) continue;
    const int col = c * 4;
    float gm[4] = {1.f, 1.f, 1.f, 1.f}, bt[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.gamma) {
      const float4 t = *reinterpret_cast<const float4*>(a.gamma + col);
      gm[0] = t.x; gm[1] = t.y; gm[2] = t.z; gm[3] = t.w;
    }
    if (a.beta) {
      const float4 t = *reinterpret_cast<const float4*>(a.beta + col);
      bt[0] = t.x; bt[1] = t.y; bt[2] = t.z; bt[3] = t.w;
    }
    const float xv[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
    float n[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) n[e] = (xv[e] - mean) * rstd * gm[e] + bt[e];
    if (BF16) {
      const uint16_t* u = static_cast<const uint16_t*>(a.u) + row * d + col;
      const uint2 ur = *reinterpret_cast<const uint2*>(u);
      const float u0 = bf2f(ur.x & 0xffff), u1 = bf2f(ur.x >> 16);
      const float u2 = bf2f(ur.y & 0xffff), u3 = bf2f(ur.y >> 16);
      uint2 o;
      o.x = pack_bf16x2(n[0] * u0, n[1] * u1);
      o.y = pack_bf16x2(n[2] * u2, n[3] * u3);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.g) + row * d + col) = o;
    } else {
      const float4 ur = *reinterpret_cast<const float4*>(static_cast<const float*>(a.u) + row * d + col);
      *reinterpret_cast<float4*>(static_cast<float*>(a.g) + row * d + col) =
          make_float4(n[0] * ur.x, n[1] * ur.y, n[2] * ur.z, n[3] * ur.w);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int64_t id = a.ids[t];
  const int act = a.acts[t];
  const bool ok = id >= 0 && id < a.num_items && act >= 0 && act < a.num_actions;
  const int d = a.d;
  if (BF16) {
    const uint16_t* it = static_cast<const uint16_t*>(a.item);
    const uint16_t* ac = static_cast<const uint16_t*>(a.action);
    uint16_t* x = static_cast<uint16_t*>(a.x) + t * d;
    for (int c = lane * 8; c < d; c += 64 * 8) {
      uint4 o;
      if (ok) {
        const uint4 ri = *reinterpret_cast<const uint4*>(it + id * d + c);
        const uint4 ra = *reinterpret_cast<const uint4*>(ac + static_cast<int64_t>(act) * d + c);
        const uint32_t wi[4] = {ri.x, ri.y, ri.z, ri.w};
        const uint32_t wa[4] = {ra.x, ra.y, ra.z, ra.w};
        uint32_t wo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wo[e] = pack_bf16x2(bf2f(wi[e] & 0xffff) + bf2f(wa[e] & 0xffff),
                              bf2f(wi[e] >> 16) + bf2f(wa[e] >> 16));
        o = make_uint4(wo[0], wo[1], wo[2], wo[3]);
      } else {
        o = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);  // bf16 NaN
      }
      *reinterpret_cast<uint4*>(x + c) = o;
    }
  } else {
    const float* it = static_cast<const float*>(a.item);
    const float* ac = static_cast<const float*>(a.action);
    float* x = static_cast<float*>(a.x) + t * d;
    for (int c = lane * 4; c < d; c += 64 * 4) {
      float4 o;
      if (ok) {
        const float4 ri = *reinterpret_cast<const float4*>(it + id * d + c);
        const float4 ra = *reinterpret_cast<const float4*>(ac + static_cast<int64_t>(act) * d + c);
        o = make_float4(ri.x + ra.x, ri.y + ra.y, ri.z + ra.z, ri.w + ra.w);
      } else {
        const float nan = __builtin_nanf("");
        o = make_float4(nan, nan, nan, nan);
      }
      *reinterpret_cast<float4*>(x + c) = o;
    }
  }
}

}  // namespace

hipError_t launch_norm_gate_bf16(const NormGateArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  hipLaunchKernelGGL(norm_gate_kernel<true>, dim3(static_cast<unsigned>((a.M + 3) / 4)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_gate_f32(const NormGateArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  hipLaunchKernelGGL(norm_gate_kernel<false>, dim3(static_cast<unsigned>((a.M + 3) / 4)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_embed_bf16(const EmbedArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<true>, dim3(static_cast<unsigned>((a.T + 3) / 4)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_embed_f32(const EmbedArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<false>, dim3(static_cast<unsigned>((a.T + 3) / 4)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
