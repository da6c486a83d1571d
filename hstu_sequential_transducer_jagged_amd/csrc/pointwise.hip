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

template <bool BF16>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int d = a.d;
  if (BF16) {
    uint2 ur[1][kNgMaxChunks];
    load_u_chunks_bf16(static_cast<const uint16_t*>(a.u) + row * d, d, lane, ur[0]);
    const float* const avr[1] = {a.av + row * d};
    uint16_t* const g[1] = {static_cast<uint16_t*>(a.g) + row * d};
    norm_gate_rows_bf16<1>(avr, ur, g, d, a.eps, a.gamma, a.beta, lane);
  } else {
    norm_gate_row_f32(a.av + row * d, static_cast<const float*>(a.u) + row * d,
                      static_cast<float*>(a.g) + row * d, d, a.eps, a.gamma, a.beta, lane);
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
