// Jagged causal SiLU attention (spatial aggregation) for gfx950.
//
// Per head h of every sequence b ("万亿参数推荐大模型：HSTU 架构如何超越传统
// Self-Attention" §2.1, second equation):
//   AV_i = sum_{j visible} SiLU(alpha q_i.k_j + rab(i, j)) v_j
// with no softmax, no running max and no row sum ("HSTU：Scaling Law 的首次
// 探索" §7.1.4, innovation 1). rab(i, j) = pos_bias[p_i - p_j + n_max - 1] +
// time_bias[min(nb-1, floor(log2(|t_i - t_j| + 1)))] (§7.1.4 innovation 2;
// bucket of the time difference as in eq. 6.2.6 of "6.2. HSTU的工程突破").
// Visibility: cache rows always; own key j for own query i iff j <= i and
// (j is not a target or j == i).
//
// bf16 kernel design (head_dim 64):
//  * one workgroup = one 64-row query tile of one sequence and HPB heads, one
//    wave per head; the relative bias is shared by all heads, so the block
//    computes each 64 x 32 bias tile once and every wave reads it from LDS
//    as the initial accumulator of its Q.K MFMA (the bias add is free);
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the accumulator layout of S^T
//    (lane = query, 4 consecutive keys) is directly the A-operand layout of
//    the S.V MFMA, so P never leaves registers;
//  * alpha is folded out of the inner loop: the block works on
//    S' = q.k + rab/alpha and evaluates P' = S' / (1 + 2^(-alpha log2(e) S'))
//    (= SiLU(alpha S') / alpha), scaling the output by alpha once at the end;
//    masked pairs get a bias that drives 2^(...) to +inf, i.e. P' = 0;
//  * key tiles entirely above the diagonal are never visited (loop bound);
//    key tiles of other targets are skipped; no softmax statistics exist.
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

constexpr int kBM = 64;   // query rows per workgroup
constexpr int kBN = 32;   // keys per step
constexpr int kDH = 64;   // head dim of the bf16 kernel

__device__ __forceinline__ int time_bucket(int64_t dt, int nb) {
  uint64_t a = dt < 0 ? (0ull - static_cast<uint64_t>(dt)) : static_cast<uint64_t>(dt);
  a += 1ull;  // |dt| + 1 >= 1 (wraps only for |dt| = 2^64-1, impossible for int64)
  int b = 63 - __clzll(static_cast<long long>(a));
  return b < nb - 1 ? b : nb - 1;
}

// Key-space helpers: key index kk in [0, nc + L): cache rows first.
struct SeqInfo {
  int64_t s;     // first own token row
  int L;         // own length
  int m;         // number of targets (last m own tokens)
  int64_t cs;    // first cache row
  int nc;        // cache length
};

__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b) {
  SeqInfo si;
  si.s = a.offsets[b];
  si.L = static_cast<int>(a.offsets[b + 1] - si.s);
  int m = a.num_targets ? a.num_targets[b] : 0;
  si.m = m < 0 ? 0 : (m > si.L ? si.L : m);
  if (a.c_offsets) {
    si.cs = a.c_offsets[b];
    si.nc = static_cast<int>(a.c_offsets[b + 1] - si.cs);
  } else {
    si.cs = 0;
    si.nc = 0;
  }
  return si;
}

__device__ __forceinline__ float silu_scaled(float s, float exp_scale) {
  const float e = __builtin_amdgcn_exp2f(s * exp_scale);
  return s * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int HPB>
__global__ __launch_bounds__(64 * HPB) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = 64 * HPB;
  constexpr int ROW = HPB * kDH + 8;        // LDS row stride (bf16), +16 B pad
  constexpr int CPR = HPB * kDH / 8;        // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kBN * ROW];
  __shared__ __attribute__((aligned(16))) float sBias[8 * 64 * 4];
  __shared__ float sTime[64];

  const int seq = blockIdx.x;
  const int n_qt = (a.max_seq_len + kBM - 1) / kBM;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.y);   // heaviest tiles first
  const SeqInfo si = seq_info(a, seq);
  const int q0 = qt * kBM;
  if (q0 >= si.L) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int d = a.d_model;
  const int col0 = blockIdx.z * HPB * kDH;
  const int h_col = col0 + wave * kDH;
  const float inv_alpha = 1.0f / a.alpha;
  const float exp_scale = -a.alpha * 1.4426950408889634f;
  const float mask_raw = -1.0e30f * inv_alpha;

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ CK = static_cast<const uint16_t*>(a.ck);
  const uint16_t* __restrict__ CV = static_cast<const uint16_t*>(a.cv);

  for (int i = tid; i < 64; i += NT) sTime[i] = i < a.nb ? a.time_bias[i] * inv_alpha : 0.0f;

  // Q fragments (B operand of S^T = K Q^T): lane -> query l16, 8 dims at 8g.
  bf16x8 qf[4][2];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int qi = q0 + qb * 16 + l16;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (qi < si.L)
        raw = *reinterpret_cast<const uint4*>(Q + (si.s + qi) * d + h_col + c * 32 + 8 * g);
      qf[qb][c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int q_hi = min(q0 + kBM, si.L);        // exclusive bound of own queries
  const int nkeys = si.nc + q_hi;                // keys any query of the tile may see
  const int nkt = (nkeys + kBN - 1) / kBN;
  const int first_tgt = si.L - si.m;

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBN;
    const int own_lo = k0 - si.nc;
    // A tile made only of targets that are not queries of this block is
    // invisible to every query of the block.
    if (own_lo >= 0 && own_lo >= first_tgt && own_lo + kBN <= q0) continue;

    __syncthreads();  // previous step's readers are done with sK/sV/sBias

    // ---- stage K and V rows [k0, k0 + kBN) of this head group into LDS ----
    for (int c = tid; c < kBN * CPR; c += NT) {
      const int r = c / CPR;
      const int cc = c - r * CPR;
      const int kk = k0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kk < nkeys) {
        const int64_t off = (kk < si.nc ? (si.cs + kk) : (si.s + kk - si.nc)) * d + col0 + cc * 8;
        const uint16_t* kp = kk < si.nc ? CK : K;
        const uint16_t* vp = kk < si.nc ? CV : V;
        kv = *reinterpret_cast<const uint4*>(kp + off);
        vv = *reinterpret_cast<const uint4*>(vp + off);
      }
      *reinterpret_cast<uint4*>(&sK[r * ROW + cc * 8]) = kv;
      *reinterpret_cast<uint4*>(&sV[r * ROW + cc * 8]) = vv;
    }

    // ---- bias tile, stored in the S^T accumulator layout ----
    // slot = (kb*4 + qb)*64 + lane: query qb*16 + lane%16, keys kb*16 + 4(lane/16) + r
    for (int slot = tid; slot < 512; slot += NT) {
      const int tile = slot >> 6;
      const int l = slot & 63;
      const int kb = tile >> 2;
      const int qb = tile & 3;
      const int qi = q0 + qb * 16 + (l & 15);
      const int kbase = k0 + kb * 16 + 4 * (l >> 4);
      float bv[4];
      const bool qvalid = qi < si.L;
      const int pq = si.nc + (qi < first_tgt ? qi : first_tgt);
      const int64_t tq = qvalid ? a.ts[si.s + qi] : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kbase + r;
        bool vis = false;
        int pk = 0;
        int64_t tk = 0;
        if (qvalid && kk < nkeys) {
          if (kk < si.nc) {
            vis = true;
            pk = kk;
            tk = a.c_ts[si.cs + kk];
          } else {
            const int j = kk - si.nc;
            vis = (j <= qi) && (j < first_tgt || j == qi);
            pk = si.nc + (j < first_tgt ? j : first_tgt);
            tk = a.ts[si.s + j];
          }
        }
        float b = mask_raw;
        if (vis) {
          int pidx = pq - pk + a.pos_center;
          pidx = pidx < 0 ? 0 : (pidx >= a.pos_len ? a.pos_len - 1 : pidx);
          b = a.pos_bias[pidx] * inv_alpha + sTime[time_bucket(tq - tk, a.nb)];
        }
        bv[r] = b;
      }
      *reinterpret_cast<float4*>(&sBias[slot * 4]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
    }
    __syncthreads();

    // ---- S^T = K Q^T + bias (per 16-key x 16-query tile), SiLU, P.V ----
    bf16x8 kf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        kf[kb][c] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&sK[(kb * 16 + l16) * ROW + wave * kDH + c * 32 + 8 * g]));

    bf16x8 pf[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      uint32_t pk[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 st = *reinterpret_cast<const f32x4*>(&sBias[((kb * 4 + qb) * 64 + lane) * 4]);
        st = mfma_16x16x32(kf[kb][0], qf[qb][0], st);
        st = mfma_16x16x32(kf[kb][1], qf[qb][1], st);
        pk[kb * 2 + 0] = pack_bf16x2(silu_scaled(st[0], exp_scale), silu_scaled(st[1], exp_scale));
        pk[kb * 2 + 1] = pack_bf16x2(silu_scaled(st[2], exp_scale), silu_scaled(st[3], exp_scale));
      }
      pf[qb] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }

#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      // B operand: the same 8 keys as P's A operand (4g..4g+3, 16+4g..16+4g+3),
      // column dt*16 + lane%16 of this head.
      const uint16_t* vcol = &sV[wave * kDH + dt * 16 + l16];
      u16x8 vr;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = (i < 4) ? (4 * g + i) : (16 + 4 * g + (i - 4));
        vr[i] = vcol[key * ROW];
      }
      const bf16x8 vf = __builtin_bit_cast(bf16x8, vr);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) acc[qb][dt] = mfma_16x16x32(pf[qb], vf, acc[qb][dt]);
    }
  }

  // ---- write AV (fp32): lane -> queries qb*16 + 4g + r, column dt*16 + lane%16 ----
  float* __restrict__ out = a.av;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = q0 + qb * 16 + 4 * g + r;
      if (qi < si.L) {
        float* row = out + (si.s + qi) * d + h_col + l16;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) row[dt * 16] = acc[qb][dt][r] * a.alpha;
      }
    }
}

// fp32 kernel: one thread per query row, plain FMA loops, exact expf and IEEE
// division. It serves the fp32 dtype (small workloads).
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int seq = blockIdx.x;
  const int qt = blockIdx.y;
  const int h = blockIdx.z;
  const SeqInfo si = seq_info(a, seq);
  const int qi = qt * 64 + threadIdx.x;
  if (qt * 64 >= si.L) return;
  const bool qvalid = qi < si.L;
  const int d = a.d_model;
  const float* Q = static_cast<const float*>(a.q);
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  const float* CK = static_cast<const float*>(a.ck);
  const float* CV = static_cast<const float*>(a.cv);
  const int first_tgt = si.L - si.m;
  float qv[DH], acc[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qv[c] = qvalid ? Q[(si.s + qi) * d + h * DH + c] : 0.0f;
    acc[c] = 0.0f;
  }
  const int pq = si.nc + (qi < first_tgt ? qi : first_tgt);
  const int64_t tq = qvalid ? a.ts[si.s + qi] : 0;
  const int q_hi = min(qt * 64 + 64, si.L);
  const int nkeys = si.nc + q_hi;
  for (int kk = 0; kk < nkeys; ++kk) {
    const bool cache = kk < si.nc;
    const int j = kk - si.nc;
    const bool vis = qvalid && (cache || ((j <= qi) && (j < first_tgt || j == qi)));
    const int64_t row = cache ? (si.cs + kk) : (si.s + j);
    const float* kr = (cache ? CK : K) + row * d + h * DH;
    const float* vr = (cache ? CV : V) + row * d + h * DH;
    if (!vis) continue;
    float dot = 0.0f;
#pragma unroll
    for (int c = 0; c < DH; ++c) dot = fmaf(qv[c], kr[c], dot);
    const int pk = cache ? kk : si.nc + (j < first_tgt ? j : first_tgt);
    const int64_t tk = cache ? a.c_ts[si.cs + kk] : a.ts[si.s + j];
    int pidx = pq - pk + a.pos_center;
    pidx = pidx < 0 ? 0 : (pidx >= a.pos_len ? a.pos_len - 1 : pidx);
    const float s = a.alpha * dot + a.pos_bias[pidx] + a.time_bias[time_bucket(tq - tk, a.nb)];
    const float w = s / (1.0f + expf(-s));
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] = fmaf(w, vr[c], acc[c]);
  }
  if (qvalid) {
#pragma unroll
    for (int c = 0; c < DH; ++c) a.av[(si.s + qi) * d + h * DH + c] = acc[c];
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.max_seq_len + kBM - 1) / kBM;
  if (a.num_seqs == 0 || n_qt == 0) return hipSuccess;
  int hpb = 1;
  for (int c : {8, 4, 2, 1})
    if (a.num_heads % c == 0) { hpb = c; break; }
  dim3 grid(a.num_seqs, n_qt, a.num_heads / hpb);
  switch (hpb) {
    case 8: hipLaunchKernelGGL(attn_bf16_kernel<8>, grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_bf16_kernel<2>, grid, dim3(128), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_bf16_kernel<1>, grid, dim3(64), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.max_seq_len + 63) / 64;
  if (a.num_seqs == 0 || n_qt == 0) return hipSuccess;
  dim3 grid(a.num_seqs, n_qt, a.num_heads);
  if (a.head_dim == 32)
    hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
