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
// layernorm: the optional input norm before f1 (the block diagram's Norm1),
//   Y = LayerNorm_d(X) * gamma + beta; same layout and reductions as
//   norm_gate, reading bf16 or fp32 X.
//
// linear_bias_tables: the position and time tables of the parameter-free
//   bias of "6.2. HSTU的工程突破" eq. 6.2.6, -m_p (p_i - p_j) - m_t bucket.
//
// cache_concat: appends a later request's K/V rows to a user's cached ones
//   (M-FALCON caching across requests, "HSTU：Scaling Law 的首次探索"
//   §7.1.5); one wave copies one output row with 16-byte accesses.
//
// embed: X[t] = item_emb[id_t] + action_emb[a_t], the action-oriented token
//   of "6.2. HSTU的工程突破" eq. 6.2.2. One wavefront per token, 16-byte
//   gathers of the two rows, fp32 add, one rounding.
#include <algorithm>

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

// One wave per row: lane owns the 4-element chunks lane + 64 i (d <= 1024).
template <bool BF16>
__global__ __launch_bounds__(256) void layernorm_kernel(LayerNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int d = a.d;
  const int nchunk = d >> 2;
  float4 x[kNgMaxChunks];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    x[i] = make_float4(0, 0, 0, 0);
    if (c < nchunk) {
      if (BF16) {
        const uint2 r = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.x) + row * d)[c];
        x[i] = make_float4(bf2f(r.x & 0xffff), bf2f(r.x >> 16), bf2f(r.y & 0xffff), bf2f(r.y >> 16));
      } else {
        x[i] = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + row * d)[c];
      }
    }
    s += (x[i].x + x[i].y) + (x[i].z + x[i].w);
  }
  const float inv_d = 1.0f / static_cast<float>(d);
  const float mean = wave_sum(s) * inv_d;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    if (lane + 64 * i < nchunk) {
      const float a0 = x[i].x - mean, a1 = x[i].y - mean, a2 = x[i].z - mean, a3 = x[i].w - mean;
      ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) * inv_d + a.eps);
#pragma unroll
  for (int i = 0; i < kNgMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c >= nchunk) continue;
    const int col = c * 4;
    float4 gm = make_float4(1.f, 1.f, 1.f, 1.f), bt = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.gamma) gm = *reinterpret_cast<const float4*>(a.gamma + col);
    if (a.beta) bt = *reinterpret_cast<const float4*>(a.beta + col);
    const float n0 = (x[i].x - mean) * rstd * gm.x + bt.x;
    const float n1 = (x[i].y - mean) * rstd * gm.y + bt.y;
    const float n2 = (x[i].z - mean) * rstd * gm.z + bt.z;
    const float n3 = (x[i].w - mean) * rstd * gm.w + bt.w;
    if (BF16) {
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + row * d)[c] =
          make_uint2(pack_bf16x2(n0, n1), pack_bf16x2(n2, n3));
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(a.y) + row * d)[c] = make_float4(n0, n1, n2, n3);
    }
  }
}

// pos_len = 2 n_max - 1 entries, entry i <-> p_i - p_j = i - (n_max - 1)
__global__ __launch_bounds__(256) void linear_bias_tables_kernel(float m_p, float m_t, int pos_len,
                                                                 int num_buckets, int pairs, float* pos,
                                                                 float* time) {
  const int half = (pos_len - 1) / 2;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < pos_len; i += gridDim.x * 256)
    pos[i] = -m_p * static_cast<float>(i - half);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < pairs * num_buckets; i += 256)
      time[i] = -m_t * static_cast<float>(i % num_buckets);
}

__global__ __launch_bounds__(256) void cache_concat_kernel(CacheConcatArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid <= a.B) a.out_off[gid] = a.a_off[gid] + a.n_off[gid];
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  // sequence b of output row r: the last b with a_off[b] + n_off[b] <= r
  int lo = 0, hi = a.B;   // invariant: start(lo) <= r < start(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.a_off[mid] + a.n_off[mid] <= r) lo = mid; else hi = mid;
  }
  const int64_t k = r - (a.a_off[lo] + a.n_off[lo]);   // row within the sequence
  const int64_t na = a.a_off[lo + 1] - a.a_off[lo];
  bool from_a = k < na;
  if (a.a_T == 0) from_a = false;   // an empty input may come with NULL pointers
  if (a.n_T == 0) from_a = true;
  // (clamped: offsets that break their contract never lead outside the inputs)
  const int64_t src = from_a ? min(max(a.a_off[lo] + k, int64_t{0}), a.a_T - 1)
                             : min(max(a.n_off[lo] + (k - na), int64_t{0}), a.n_T - 1);
  const uint8_t* sk = static_cast<const uint8_t*>(from_a ? a.a_k : a.n_k) + src * a.row_bytes;
  const uint8_t* sv = static_cast<const uint8_t*>(from_a ? a.a_v : a.n_v) + src * a.row_bytes;
  uint8_t* dk = static_cast<uint8_t*>(a.out_k) + r * a.row_bytes;
  uint8_t* dv = static_cast<uint8_t*>(a.out_v) + r * a.row_bytes;
  for (int c = lane * 16; c < a.row_bytes; c += 64 * 16) {
    *reinterpret_cast<uint4*>(dk + c) = *reinterpret_cast<const uint4*>(sk + c);
    *reinterpret_cast<uint4*>(dv + c) = *reinterpret_cast<const uint4*>(sv + c);
  }
  if (lane == 0) a.out_ts[r] = from_a ? a.a_ts[src] : a.n_ts[src];
}

// One wave per row, 8-byte accesses.
__global__ __launch_bounds__(256) void gather_rows_kernel(int64_t n, int row_bytes, const int64_t* rows,
                                                          int64_t src_rows, const uint8_t* src,
                                                          uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int64_t sr = min(max(rows[r], int64_t{0}), src_rows - 1);
  const uint8_t* s = src + sr * row_bytes;
  uint8_t* d = dst + r * row_bytes;
  for (int c = lane * 8; c < row_bytes; c += 64 * 8)
    *reinterpret_cast<uint2*>(d + c) = *reinterpret_cast<const uint2*>(s + c);
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

hipError_t launch_layernorm_bf16(const LayerNormArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  hipLaunchKernelGGL(layernorm_kernel<true>, dim3(static_cast<unsigned>((a.M + 3) / 4)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_layernorm_f32(const LayerNormArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  hipLaunchKernelGGL(layernorm_kernel<false>, dim3(static_cast<unsigned>((a.M + 3) / 4)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_linear_bias_tables(float m_p, float m_t, int pos_len, int num_buckets, int pairs,
                                     float* pos, float* time, hipStream_t s) {
  const int grid = (pos_len + 255) / 256;
  hipLaunchKernelGGL(linear_bias_tables_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, s, m_p, m_t,
                     pos_len, num_buckets, pairs, pos, time);
  return hipGetLastError();
}

hipError_t launch_gather_rows(int64_t n, int row_bytes, const int64_t* rows, int64_t src_rows,
                              const void* src, void* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, s, n,
                     row_bytes, rows, src_rows, static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_cache_concat(const CacheConcatArgs& a, hipStream_t s) {
  // enough blocks for every output row (4 per block) and for the B + 1 offsets
  const int64_t blocks = std::max<int64_t>((a.rows + 3) / 4, (static_cast<int64_t>(a.B) + 1 + 255) / 256);
  hipLaunchKernelGGL(cache_concat_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
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
