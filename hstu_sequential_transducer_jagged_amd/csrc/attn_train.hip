// Attention of one HSTU layer for training, fp32 on the matrix cores
// (v_mfma_f32_16x16x4_f32). Plain causal attention over the batch's own
// tokens, as "HSTU：Scaling Law 的首次探索" §7.1.5 trains it: per head
//   S = alpha Q K^T + rab,  P = SiLU(S) . M,  AV = P V
// ("万亿参数推荐大模型…" §2.1 second equation), and its backward
//   dP = dAV V^T,  dS = dP . SiLU'(S) . M,  dV = P^T dAV,
//   dQ = alpha dS K,  dK = alpha dS^T Q,  d rab(i, j) += dS(i, j).
//
// Three kernels share one structure. A wave owns 32 rows of one head (query
// rows for the forward and dQ, key rows for dK/dV), keeps their operands in
// registers, and walks the visible 32-row blocks of the other side:
//   * score-shaped products over the 32x32 block (S, and dP for the
//     backward), as 2x2 tiles of 16x16, whose accumulators put one query
//     or key per lane and 4 rows of the other side in each tile's registers;
//   * the pointwise step in those registers (bias, SiLU, mask, dS);
//   * the second product(s), where each accumulator register is exactly the
//     B operand of a 16x16x4 step over 4 rows of that side.
// The contraction order of every product is free, so each operand is loaded
// in the order that suits its layout: float4 runs along the head dimension
// for the row-per-lane operands, and whole rows across the lanes for the
// dimension-per-lane ones. A workgroup holds one wave per head of the same
// 32 rows (up to four heads), so its waves have identical trip counts.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2eT = 1.4426950408889634f;
// Waves (heads) per workgroup, at most. Four-wave workgroups let two or three
// of them share a CU and drift out of step, so that one's matrix work
// overlaps another's pointwise step; with one eight-wave workgroup per CU
// the forward ran 18 % and the backward 10 % slower.
// (The kernels keep a 512-thread launch bound all the same: it holds them to
// 256 registers, two waves per SIMD.)
constexpr int kMaxWaves = 4;
// Entries of the workgroup's LDS accumulator of position-bias gradients
// (position differences -31 .. kPosCap-32); larger differences are added to
// global memory directly.
constexpr int kPosCap = 16384 + 64;

// 16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16]; accumulator
// register r of lane l is D[4 (l/16) + r][l%16]. (The 32x32x2 form runs at
// half this rate on gfx950.)
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoid_t(float s) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2eT * s));
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Time bucket in 32-bit arithmetic. A time t is kept as its offset from a
// reference time, biased by 2^31 (mod 2^64). When every time a block uses
// gives an offset below 2^32 - 1, the difference of two offsets is the
// wrapped 64-bit difference of their times, and its magnitude plus one fits
// in 32 bits, so time_bucket32 returns what time_bucket64 returns for that
// difference. The test is made per block for the whole wave.
__device__ __forceinline__ uint64_t time_off(int64_t t, int64_t tref) {
  return static_cast<uint64_t>(t) - static_cast<uint64_t>(tref) + (uint64_t{1} << 31);
}
__device__ __forceinline__ bool time_fits32(uint64_t off) { return off < 0xffffffffull; }
// The bf16 kernels look the time table up by a key, 31 - floor(log2(|dt| + 1))
// in -32 .. 31, from which the bucket is min(31 - key, nb - 1): LDS tables
// indexed by key + 32 hold the clamp, so the 32-bit path costs an absolute
// difference and a leading-zero count per pair.
__device__ __forceinline__ int time_key32(uint32_t x, uint32_t y) {
  const uint32_t m = (x > y ? x - y : y - x) + 1u;   // |dt| + 1 <= 2^32 - 1
  return __builtin_clz(m);
}
__device__ __forceinline__ int time_key64(int64_t dt) {
  uint64_t m = dt < 0 ? (0ull - static_cast<uint64_t>(dt)) : static_cast<uint64_t>(dt);
  m += 1ull;
  return __clzll(static_cast<long long>(m)) - 32;
}

__device__ __forceinline__ float comp(const float4& v, int e) {
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// Row-per-lane operand of a product over the head dimension: lane (row, g)
// holds columns 16u + 4g + e (u < DH/16, e < 4) of its row, so that step
// t = 4u + e contracts columns 16u + 4g' + e over the lane groups g'.
template <int DH>
__device__ __forceinline__ void load_rowop(const float* row, int g, float4 (&o)[DH / 16]) {
#pragma unroll
  for (int u = 0; u < DH / 16; ++u) o[u] = *reinterpret_cast<const float4*>(row + 16 * u + 4 * g);
}

// Dimension-per-lane operand: the NCT = DH/16 columns NCT*lc .. NCT*lc+NCT-1
// of one row, so that output tile ct, row lc is column NCT*lc + ct.
template <int NCT>
struct ColOp {
  float v[NCT];
};
template <int NCT>
__device__ __forceinline__ ColOp<NCT> load_colop(const float* row, int lc) {
  ColOp<NCT> o;
  if constexpr (NCT == 4) {
    const float4 x = *reinterpret_cast<const float4*>(row + 4 * lc);
    o.v[0] = x.x; o.v[1] = x.y; o.v[2] = x.z; o.v[3] = x.w;
  } else {
    const float2 x = *reinterpret_cast<const float2*>(row + 2 * lc);
    o.v[0] = x.x; o.v[1] = x.y;
  }
  return o;
}

// Stores the NCT x 2 output tiles of one lane: tile (ct, bt), register r is
// output row i = 4g + r -> column NCT*i + ct, of the lane's row 16 bt + lc.
// out points at row 16*0 + lc, head column 0; ld is the row stride.
template <int NCT>
__device__ __forceinline__ void store_tiles(float* out, int64_t ld, const f32x4 (&acc)[NCT][2], int g,
                                            float scale, bool ok0, bool ok1) {
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    if (!(bt == 0 ? ok0 : ok1)) continue;
    float* row = out + bt * 16 * ld;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = NCT * (4 * g + r);
      if constexpr (NCT == 4) {
        float4 x;
        x.x = acc[0][bt][r] * scale; x.y = acc[1][bt][r] * scale;
        x.z = acc[2][bt][r] * scale; x.w = acc[3][bt][r] * scale;
        *reinterpret_cast<float4*>(row + c) = x;
      } else {
        float2 x;
        x.x = acc[0][bt][r] * scale; x.y = acc[1][bt][r] * scale;
        *reinterpret_cast<float2*>(row + c) = x;
      }
    }
  }
}

struct Place {
  int seq, blk, h;
};

// Workgroup -> (sequence, 32-row block, head of this wave). Blocks are taken
// heaviest first: descending for query blocks (more keys below them),
// ascending for key blocks (more queries above them). Workgroups go to the
// XCDs round-robin, so with the (sequence, head group) index alone each XCD
// would keep the same few sequences for the whole launch, and the cost of a
// sequence grows with its squared length; the index is rotated by the block
// row so that every sequence's rows spread over all XCDs.
__device__ __forceinline__ Place place(const BwdAttnArgs& a, bool descending, int wave, int nw) {
  const int hgs = a.num_heads / nw;
  const int nblk = (a.max_seq_len + 31) >> 5;
  const int per = a.num_seqs * hgs;
  const int b = static_cast<int>(blockIdx.x) / per;
  int rem = static_cast<int>(blockIdx.x) - b * per;
  rem = (rem + b) % per;
  Place p;
  p.blk = descending ? nblk - 1 - b : b;
  p.seq = rem / hgs;
  p.h = (rem - p.seq * hgs) * nw + wave;
  return p;
}

// Forward (FWD: AV) or dQ with the bias-table gradients, for the 32 query
// rows of one block (two 16-row tiles) and one head per wave. LONG: some
// position differences may lie beyond the LDS accumulator (sequences longer
// than kPosCap - 64); those are added to global memory one by one.
template <int DH, bool FWD, bool LONG = false>
__global__ __launch_bounds__(512) void attn_train_q_kernel(BwdAttnArgs a) {
  constexpr int NU = DH / 16, NCT = DH / 16;
  __shared__ float s_gpos[FWD ? 1 : kPosCap];
  __shared__ float s_tval[64], s_tgrad[64];
  __shared__ float s_win[kMaxWaves][64];
  __shared__ int64_t s_ts[kMaxWaves][32];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, g = lane >> 4;
  const Place pl = place(a, true, wave, nw);
  const int64_t s0 = a.offsets[pl.seq];
  const int L = static_cast<int>(a.offsets[pl.seq + 1] - s0);
  const int q0 = pl.blk * 32;
  if (q0 >= L) return;   // the whole workgroup: same sequence and block
  const int range = min(q0 + 63, kPosCap);   // LDS entries d + 31 this block can touch
  if (!FWD) {
    for (int e = tid; e < range; e += blockDim.x) s_gpos[e] = 0.0f;
    if (tid < 64) s_tgrad[tid] = 0.0f;
  }
  if (tid < 64) s_tval[tid] = tid < a.nb ? a.time_bias[tid] : 0.0f;
  __syncthreads();

  const int d = a.d_model;
  // this sequence's rows of the head; row offsets within a sequence are int32
  const int64_t base = s0 * d + pl.h * DH;
  const float* Ks = a.k + base;
  const float* Vs = a.v + base;
  const float* Cs = FWD ? Vs : Ks;   // operand of the second product
  const int64_t* Ts = a.ts + s0;
  // query tiles: rows q0 + lc and q0 + 16 + lc
  float4 qr[2][NU], dr[2][NU];
  int64_t tq[2];
  bool qv[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = min(q0 + 16 * qt + lc, L - 1);
    qv[qt] = q0 + 16 * qt + lc < L;
    load_rowop<DH>(a.q + base + qrow * d, g, qr[qt]);
    if (!FWD) load_rowop<DH>(a.dav + base + qrow * d, g, dr[qt]);
    tq[qt] = Ts[qrow];
  }
  float* win = s_win[wave];
  int64_t* kts = s_ts[wave];
  f32x4 acc[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct][0] = acc[ct][1] = f32x4{};
  // time-bucket gradients: per lane and query tile the keys ascend, so runs
  // of one bucket are summed in registers and added to LDS when the bucket
  // changes (starting from bucket 0 with nothing summed)
  int tb_cur[2] = {0, 0};
  float tg_cur[2] = {0.0f, 0.0f};
  // position-bias window of block kb: entry e <-> difference q0 - 32 kb - 31 + e;
  // the window value and the key timestamp of this lane are fetched a block ahead
  float wv = a.pos_bias[clampi(a.pos_center + q0 - 31 + lane, 0, a.pos_len - 1)];
  int64_t tsv = Ts[min(lane & 31, L - 1)];

  for (int kb = 0; kb <= pl.blk; ++kb) {
    const int j0 = kb * 32, D = q0 - j0;
    win[lane] = wv;
    if (lane < 32) kts[lane] = tsv;
    wv = a.pos_bias[clampi(a.pos_center + D - 63 + lane, 0, a.pos_len - 1)];
    tsv = Ts[min(j0 + 32 + (lane & 31), L - 1)];
    float4 kr[2][NU], vr[2][NU];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int krow = min(j0 + 16 * kt + lc, L - 1);
      load_rowop<DH>(Ks + krow * d, g, kr[kt]);
      if (!FWD) load_rowop<DH>(Vs + krow * d, g, vr[kt]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // S^T = K Q^T (rows: keys, columns: queries); dP^T = V dAV^T
    f32x4 sacc[2][2], pacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) sacc[kt][qt] = pacc[kt][qt] = f32x4{};
#pragma unroll
    for (int t = 0; t < DH / 4; ++t)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          sacc[kt][qt] = mma(comp(kr[kt][t >> 2], t & 3), comp(qr[qt][t >> 2], t & 3), sacc[kt][qt]);
          if (!FWD)
            pacc[kt][qt] = mma(comp(vr[kt][t >> 2], t & 3), comp(dr[qt][t >> 2], t & 3), pacc[kt][qt]);
        }
    // the second product's operand, requested while the scores finish (it
    // takes the registers of K and V above): key row 16 kt + 4g + r
    ColOp<NCT> kc[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) kc[kt][r] = load_colop<NCT>(Cs + min(j0 + 16 * kt + 4 * g + r, L - 1) * d, lc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jr = 16 * kt + 4 * g + r;   // key row in the block
        const int64_t tk = kts[jr];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int ir = 16 * qt + lc;        // query row in the block
          const bool vis = qv[qt] && (j0 + jr <= q0 + ir);
          const int tb = time_bucket64(tq[qt] - tk, a.nb);
          const float sc = a.alpha * sacc[kt][qt][r] + win[ir - jr + 31] + s_tval[tb];
          const float sg = sigmoid_t(sc);
          if (FWD) {
            sacc[kt][qt][r] = vis ? sc * sg : 0.0f;
          } else {
            const float ds = vis ? pacc[kt][qt][r] * sg * (1.0f + sc * (1.0f - sg)) : 0.0f;
            sacc[kt][qt][r] = ds;
            // hidden pairs add zero (their index D + ir - jr + 31 >= 0 is in range)
            const int gi = D + ir - jr + 31;
            if (!LONG || gi < kPosCap)
              atomicAdd(&s_gpos[gi], ds);
            else if (vis)
              atomicAdd(&a.dpos[clampi(a.pos_center + gi - 31, 0, a.pos_len - 1)], ds);
            const bool flush = vis && tb != tb_cur[qt];
            if (flush) atomicAdd(&s_tgrad[tb_cur[qt]], tg_cur[qt]);
            tg_cur[qt] = (flush ? 0.0f : tg_cur[qt]) + ds;
            tb_cur[qt] = flush ? tb : tb_cur[qt];
          }
        }
      }
    // dQ^T += K^T dS^T (AV^T += V^T P^T): step (kt, r) contracts keys 16 kt + 4g' + r
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) acc[ct][qt] = mma(kc[kt][r].v[ct], sacc[kt][qt][r], acc[ct][qt]);
  }

  if (FWD)
    store_tiles<NCT>(a.av + (s0 + q0 + lc) * d + pl.h * DH, d, acc, g, 1.0f, qv[0], qv[1]);
  else
    store_tiles<NCT>(a.dq + (s0 + q0 + lc) * a.ld_dz + pl.h * DH, a.ld_dz, acc, g, a.alpha, qv[0], qv[1]);
  if (!FWD) {
    atomicAdd(&s_tgrad[tb_cur[0]], tg_cur[0]);
    atomicAdd(&s_tgrad[tb_cur[1]], tg_cur[1]);
    __syncthreads();
    for (int e = tid; e < range; e += blockDim.x) {
      const float gsum = s_gpos[e];
      if (gsum != 0.0f) atomicAdd(&a.dpos[clampi(a.pos_center + e - 31, 0, a.pos_len - 1)], gsum);
    }
    if (tid < a.nb && s_tgrad[tid] != 0.0f) atomicAdd(&a.dtime[tid], s_tgrad[tid]);
  }
}

// dK and dV for the 32 key rows of one block (two 16-row tiles) and one
// head per wave.
template <int DH>
__global__ __launch_bounds__(512) void attn_train_kv_kernel(BwdAttnArgs a) {
  constexpr int NU = DH / 16, NCT = DH / 16;
  __shared__ float s_tval[64];
  __shared__ float s_win[kMaxWaves][64];
  __shared__ int64_t s_ts[kMaxWaves][32];
  // V rows of each wave, parked in LDS by the lane that reads them back
  // (registers are the limit here); 16-byte padding per lane
  __shared__ float4 s_v[kMaxWaves][2][NU][64 + 1];
  __shared__ int64_t s_kts[kMaxWaves][32];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, g = lane >> 4;
  const Place pl = place(a, false, wave, nw);
  const int64_t s0 = a.offsets[pl.seq];
  const int L = static_cast<int>(a.offsets[pl.seq + 1] - s0);
  const int j0 = pl.blk * 32;
  if (j0 >= L) return;
  if (tid < 64) s_tval[tid] = tid < a.nb ? a.time_bias[tid] : 0.0f;
  __syncthreads();

  const int d = a.d_model;
  const int64_t base = s0 * d + pl.h * DH;
  const float* Qs = a.q + base;
  const float* Ds = a.dav + base;
  const int64_t* Ts = a.ts + s0;
  float4 kr[2][NU];
  bool kv[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int krow = min(j0 + 16 * kt + lc, L - 1);
    kv[kt] = j0 + 16 * kt + lc < L;
    load_rowop<DH>(a.k + base + krow * d, g, kr[kt]);
    float4 vr[NU];
    load_rowop<DH>(a.v + base + krow * d, g, vr);
#pragma unroll
    for (int u = 0; u < NU; ++u) s_v[wave][kt][u][lane] = vr[u];
  }
  if (lane < 32) s_kts[wave][lane] = Ts[min(j0 + lane, L - 1)];
  float* win = s_win[wave];
  int64_t* qts = s_ts[wave];
  f32x4 dk[NCT][2], dv[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) dk[ct][0] = dk[ct][1] = dv[ct][0] = dv[ct][1] = f32x4{};
  const int nblk = (L + 31) >> 5;
  // window entry e <-> difference 32 qb - j0 - 31 + e; fetched a block ahead
  float wv = a.pos_bias[clampi(a.pos_center - 31 + lane, 0, a.pos_len - 1)];
  int64_t tsv = Ts[min(j0 + (lane & 31), L - 1)];
  for (int qb = pl.blk; qb < nblk; ++qb) {
    const int q0 = qb * 32, D = q0 - j0;
    win[lane] = wv;
    if (lane < 32) qts[lane] = tsv;
    wv = a.pos_bias[clampi(a.pos_center + D + 1 + lane, 0, a.pos_len - 1)];
    tsv = Ts[min(q0 + 32 + (lane & 31), L - 1)];
    float4 qa[2][NU], da[2][NU], vr[2][NU];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int qrow = min(q0 + 16 * qt + lc, L - 1);
      load_rowop<DH>(Qs + qrow * d, g, qa[qt]);
      load_rowop<DH>(Ds + qrow * d, g, da[qt]);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < NU; ++u) vr[kt][u] = s_v[wave][kt][u][lane];
    __builtin_amdgcn_sched_barrier(0);
    // S = Q K^T (rows: queries, columns: keys); dP = dAV V^T
    f32x4 sacc[2][2], pacc[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sacc[qt][kt] = pacc[qt][kt] = f32x4{};
#pragma unroll
    for (int t = 0; t < DH / 4; ++t)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          sacc[qt][kt] = mma(comp(qa[qt][t >> 2], t & 3), comp(kr[kt][t >> 2], t & 3), sacc[qt][kt]);
          pacc[qt][kt] = mma(comp(da[qt][t >> 2], t & 3), comp(vr[kt][t >> 2], t & 3), pacc[qt][kt]);
        }
    // the second products' operands (in the registers of qa/da): query row 16 qt + 4g + r
    ColOp<NCT> qc[2][4], dc[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = min(q0 + 16 * qt + 4 * g + r, L - 1) * d;
        qc[qt][r] = load_colop<NCT>(Qs + row, lc);
        dc[qt][r] = load_colop<NCT>(Ds + row, lc);
      }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tk[2] = {s_kts[wave][lc], s_kts[wave][16 + lc]};
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ir = 16 * qt + 4 * g + r;   // query row in the block
        const int64_t tqr = qts[ir];
        const bool qok = q0 + ir < L;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int jr = 16 * kt + lc;        // key row in the block
          const bool vis = kv[kt] && qok && (j0 + jr <= q0 + ir);
          const int tb = time_bucket64(tqr - tk[kt], a.nb);
          const float sc = a.alpha * sacc[qt][kt][r] + win[ir - jr + 31] + s_tval[tb];
          const float sg = sigmoid_t(sc);
          sacc[qt][kt][r] = vis ? sc * sg : 0.0f;
          pacc[qt][kt][r] = vis ? pacc[qt][kt][r] * sg * (1.0f + sc * (1.0f - sg)) : 0.0f;
        }
      }
    // dV^T += dAV^T P, dK^T += Q^T dS: step (qt, r) contracts queries 16 qt + 4g' + r
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            dv[ct][kt] = mma(dc[qt][r].v[ct], sacc[qt][kt][r], dv[ct][kt]);
            dk[ct][kt] = mma(qc[qt][r].v[ct], pacc[qt][kt][r], dk[ct][kt]);
          }
  }
  store_tiles<NCT>(a.dk + (s0 + j0 + lc) * a.ld_dz + pl.h * DH, a.ld_dz, dk, g, a.alpha, kv[0], kv[1]);
  store_tiles<NCT>(a.dv + (s0 + j0 + lc) * a.ld_dz + pl.h * DH, a.ld_dz, dv, g, 1.0f, kv[0], kv[1]);
}

// ---------------------------------------------------------------------------
// The backward on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16): the same
// products, pointwise step and table gradients as above, from bf16 copies
// of Q, K, V and dAV, with P and dS rounded to bf16 as the operands of their
// products and every sum in fp32.
//
// 16x16x32: lane l supplies A[l%16][8 (l/16) + e] and B[8 (l/16) + e][l%16]
// (e < 8); accumulator register r of lane l is D[4 (l/16) + r][l%16], the
// layout of the 16x16x4 fp32 form. The score-shaped products contract the
// head dimension, so their operands are rows read straight from memory (8
// consecutive dims per lane). The second products contract the 32 rows of
// the block walked: their B operand is the accumulator itself, lane group g
// holding rows 4g + r of the first and the second 16-row tile (slots
// e = 4 t + r), and their A operand is the other side's 32 x DH block read
// back transposed from the wave's LDS copy (ds_read_b64_tr_b16: within 16
// lanes, source lane 4a + b addresses dims 4b .. 4b+3 of row a, and lane i
// receives dim i of rows 0 .. 3), which yields the same slot order.
// ---------------------------------------------------------------------------

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define HSTU_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// LDS accumulator of position-bias gradients of the bf16 dQ kernel:
// differences -31 .. kPosCapB - 32; larger ones go to global memory.
constexpr int kPosCapB = 8192 + 64;

// Row-per-lane bf16 operand over the head dimension: lane (row, g) holds
// dims 32c + 8g .. 32c + 8g + 7 of its row (c < DH / 32).
template <int NC>
__device__ __forceinline__ void load_row16(const uint16_t* row, int g, bf16x8 (&o)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
    o[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + 32 * c + 8 * g));
}

// The wave's 32 x DH block in LDS (row stride DH + 8 bf16: the four rows one
// transposing read touches start in different banks), from the row operands
// of its two 16-row tiles.
template <int DH>
__device__ __forceinline__ void stash_block(uint16_t* blk, const bf16x8 (&o)[2][DH / 32], int lc, int g) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < DH / 32; ++c)
      *reinterpret_cast<uint4*>(blk + (16 * t + lc) * (DH + 8) + 32 * c + 8 * g) =
          __builtin_bit_cast(uint4, o[t][c]);
}

// A operand of a second product, for output dims 16 ct .. 16 ct + 15: lane
// (lc, g) gets dim 16 ct + lc of block rows 4g .. 4g+3 (slots 0..3) and
// 16 + 4g .. 16 + 4g + 3 (slots 4..7).
template <int DH>
__device__ __forceinline__ bf16x8 load_block_tr(const uint16_t* blk, int ct, int lc, int g) {
  const uint16_t* p = blk + (4 * g + (lc >> 2)) * (DH + 8) + 16 * ct + 4 * (lc & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(HSTU_LDS(i16x4, p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(HSTU_LDS(i16x4, p + 16 * (DH + 8)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B operand of a second product from two accumulator tiles (slots 4t + r).
__device__ __forceinline__ bf16x8 pack_slots(const f32x4& t0, const f32x4& t1) {
  const uint4 u = make_uint4(pack_bf16x2(t0[0], t0[1]), pack_bf16x2(t0[2], t0[3]), pack_bf16x2(t1[0], t1[1]),
                             pack_bf16x2(t1[2], t1[3]));
  return __builtin_bit_cast(bf16x8, u);
}

// Output tile of a second product: accumulator register r of lane (lc, g) is
// dim 16 ct + 4g + r of row lc of the 16-row tile; one float4 per tile.
template <int NCT>
__device__ __forceinline__ void store_tiles16(float* out, int64_t ld, const f32x4 (&acc)[NCT][2], int lc, int g,
                                              float scale, bool ok0, bool ok1) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!(t == 0 ? ok0 : ok1)) continue;
    float* row = out + (16 * t + lc) * ld;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      *reinterpret_cast<float4*>(row + 16 * ct + 4 * g) =
          make_float4(acc[ct][t][0] * scale, acc[ct][t][1] * scale, acc[ct][t][2] * scale, acc[ct][t][3] * scale);
  }
}

// dQ with the bias-table gradients for the 32 query rows of one block and one
// head per wave. The position gradient sums each diagonal of a block before
// anything is added: the wave parks its dS block in LDS, lane l sums
// diagonal l (query row - key row = l - 31) and adds the sum to the position
// accumulator once. The time-bucket gradient sums runs of one bucket per
// lane in registers, as the fp32 kernel does. LONG: some position
// differences lie beyond the LDS accumulator; those are added to global
// memory.
template <int DH, bool LONG>
__global__ __launch_bounds__(512) void attn_train_dq_bf16_kernel(BwdAttnArgs a) {
  constexpr int NC = DH / 32, NCT = DH / 16;
  constexpr int DSR = 36;   // row stride of a parked dS block (16-byte rows, spread over the banks)
  __shared__ float s_gpos[kPosCapB];
  __shared__ float s_tvk[64], s_tgk[64];   // by time key + 32
  __shared__ float s_win[kMaxWaves][64];
  __shared__ int64_t s_ts[kMaxWaves][32];
  __shared__ uint32_t s_ts32[kMaxWaves][32];
  __shared__ __attribute__((aligned(16))) float s_ds[kMaxWaves][32 * DSR];
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxWaves][32 * (DH + 8)];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, g = lane >> 4;
  const Place pl = place(a, true, wave, nw);
  const int64_t s0 = a.offsets[pl.seq];
  const int L = static_cast<int>(a.offsets[pl.seq + 1] - s0);
  const int q0 = pl.blk * 32;
  if (q0 >= L) return;   // the whole workgroup: same sequence and block
  const int range = min(q0 + 63, kPosCapB);   // LDS entries d + 31 this block can touch
  const int64_t* Ts = a.ts + s0;
  for (int e = tid; e < range; e += blockDim.x) s_gpos[e] = 0.0f;
  if (tid < 64) {
    s_tgk[tid] = 0.0f;
    s_tvk[tid] = a.time_bias[min(63 - tid, a.nb - 1)];
  }
  __syncthreads();

  const int d = a.d_model;
  const int64_t base = s0 * d + pl.h * DH;
  const uint16_t* Ks = a.k16 + base;
  const uint16_t* Vs = a.v16 + base;
  uint16_t* kblk = s_k[wave];
  bf16x8 qf[2][NC], df[2][NC];
  int64_t tq[2];
  uint32_t tq32[2];
  bool qv[2];
  // times as 32-bit offsets from the block's first query time where they fit
  const int64_t tref = Ts[q0];
  bool fq = true;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = min(q0 + 16 * qt + lc, L - 1);
    qv[qt] = q0 + 16 * qt + lc < L;
    load_row16<NC>(a.q16 + base + qrow * d, g, qf[qt]);
    load_row16<NC>(a.dav16 + base + qrow * d, g, df[qt]);
    tq[qt] = Ts[qrow];
    const uint64_t off = time_off(tq[qt], tref);
    fq = fq && time_fits32(off);
    tq32[qt] = static_cast<uint32_t>(off);
  }
  const bool fast_q = __builtin_amdgcn_ballot_w64(!fq) == 0;
  float* win = s_win[wave];
  int64_t* kts = s_ts[wave];
  uint32_t* kts32 = s_ts32[wave];
  f32x4 acc[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct][0] = acc[ct][1] = f32x4{};
  // time-bucket gradients: per lane and query tile the keys ascend, so runs
  // of one time key are summed in registers and added to LDS when the key
  // changes (starting from key 31, bucket 0, with nothing summed); the
  // entries go to their buckets at the end
  const float* tvk = s_tvk + 32;
  float* tgk = s_tgk + 32;
  int tb_cur[2] = {31, 31};   // time keys
  float tg_cur[2] = {0.0f, 0.0f};
  float wv = a.pos_bias[clampi(a.pos_center + q0 - 31 + lane, 0, a.pos_len - 1)];
  int64_t tsv = Ts[min(lane & 31, L - 1)];
  // the block's K and V rows; each step requests the next block's rows into
  // the same registers once the score products and the stash have read them
  bf16x8 kf[2][NC], vf[2][NC];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int krow = min(16 * kt + lc, L - 1);
    load_row16<NC>(Ks + krow * d, g, kf[kt]);
    load_row16<NC>(Vs + krow * d, g, vf[kt]);
  }

  for (int kb = 0; kb <= pl.blk; ++kb) {
    const int j0 = kb * 32, D = q0 - j0;
    win[lane] = wv;
    const uint64_t koff = time_off(tsv, tref);
    const bool fast = fast_q && __builtin_amdgcn_ballot_w64(!time_fits32(koff)) == 0;
    if (lane < 32) {
      kts[lane] = tsv;
      kts32[lane] = static_cast<uint32_t>(koff);
    }
    wv = a.pos_bias[clampi(a.pos_center + D - 63 + lane, 0, a.pos_len - 1)];
    tsv = Ts[min(j0 + 32 + (lane & 31), L - 1)];
    // S^T = K Q^T (rows: keys, columns: queries); dP^T = V dAV^T
    f32x4 sacc[2][2], pacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        sacc[kt][qt] = pacc[kt][qt] = f32x4{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc[kt][qt] = mfma_16x16x32(kf[kt][c], qf[qt][c], sacc[kt][qt]);
          pacc[kt][qt] = mfma_16x16x32(vf[kt][c], df[qt][c], pacc[kt][qt]);
        }
      }
    // this block's keys, for the transposed reads of the second product
    stash_block<DH>(kblk, kf, lc, g);
    if (kb < pl.blk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int krow = min(j0 + 32 + 16 * kt + lc, L - 1);
        load_row16<NC>(Ks + krow * d, g, kf[kt]);
        load_row16<NC>(Vs + krow * d, g, vf[kt]);
      }
    }
    // per 16-key half: every LDS read first (key times and position-window
    // entries, then the time-table entries of the buckets), then the
    // arithmetic for every pair, masked by a select; read behind the
    // visibility test, each pair's lookups were waited for on their own
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float wq[4][2], tvq[4][2];
      int tbq[4][2];
      if (fast) {
        uint32_t tk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) tk[r] = kts32[16 * kt + 4 * g + r];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) tbq[r][qt] = time_key32(tq32[qt], tk[r]);
      } else {
        int64_t tk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) tk[r] = kts[16 * kt + 4 * g + r];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) tbq[r][qt] = time_key64(tq[qt] - tk[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) wq[r][qt] = win[16 * qt + lc - (16 * kt + 4 * g + r) + 31];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) tvq[r][qt] = tvk[tbq[r][qt]];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jr = 16 * kt + 4 * g + r;   // key row in the block
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int ir = 16 * qt + lc;        // query row in the block
          const bool vis = qv[qt] && (j0 + jr <= q0 + ir);
          const int tb = tbq[r][qt];
          const float sc = a.alpha * sacc[kt][qt][r] + wq[r][qt] + tvq[r][qt];
          const float sg = sigmoid_t(sc);
          const float dsv = pacc[kt][qt][r] * __builtin_fmaf(sc, __builtin_fmaf(-sg, sg, sg), sg);
          const float ds = vis ? dsv : 0.0f;
          sacc[kt][qt][r] = ds;
          const bool flush = vis && tb != tb_cur[qt];
          if (flush) atomicAdd(&tgk[tb_cur[qt]], tg_cur[qt]);
          tg_cur[qt] = (flush ? 0.0f : tg_cur[qt]) + ds;
          tb_cur[qt] = flush ? tb : tb_cur[qt];
        }
      }
    }
    // park dS (query row ir = 16 qt + lc, key rows 16 kt + 4g .. +3)
    float* dsw = s_ds[wave];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        *reinterpret_cast<float4*>(dsw + (16 * qt + lc) * DSR + 16 * kt + 4 * g) =
            make_float4(sacc[kt][qt][0], sacc[kt][qt][1], sacc[kt][qt][2], sacc[kt][qt][3]);
    // dQ^T += K^T dS^T over the block's 32 keys, and the position gradient:
    // lane l sums diagonal l of this wave's parked block (rows ir with key
    // row jr = ir - l + 31 in the block; hidden pairs hold dS = 0). LDS
    // accesses of one wave complete in order, so the block is read back
    // without a barrier. The K^T operand reads go out first, then the first
    // half of the diagonal reads, so that these land while the products run;
    // the second half follows the products. (Adding each pair's dS to the
    // accumulator with an LDS atomic instead, sixteen per lane and step, ran
    // 3.4 times slower.)
    bf16x8 bs[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) bs[qt] = pack_slots(sacc[0][qt], sacc[1][qt]);
    bf16x8 kt_op[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) kt_op[ct] = load_block_tr<DH>(kblk, ct, lc, g);
    float v[32];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int jr = e - lane + 31;   // in the block for ir = e in [lane - 31, lane]
      v[e] = dsw[e * DSR + min(max(jr, 0), 31)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) acc[ct][qt] = mfma_16x16x32(kt_op[ct], bs[qt], acc[ct][qt]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 16; e < 32; ++e) {
      const int jr = e - lane + 31;
      v[e] = dsw[e * DSR + min(max(jr, 0), 31)];
    }
    float pos_sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int jr = e - lane + 31;
      pos_sum += (jr >= 0 && jr < 32) ? v[e] : 0.0f;
    }
    if (lane < 63 && pos_sum != 0.0f) {
      const int gi = D + lane;   // difference D + lane - 31
      if (!LONG || gi < kPosCapB)
        atomicAdd(&s_gpos[gi], pos_sum);
      else
        atomicAdd(&a.dpos[clampi(a.pos_center + gi - 31, 0, a.pos_len - 1)], pos_sum);
    }
  }

  store_tiles16<NCT>(a.dq + (s0 + q0) * a.ld_dz + pl.h * DH, a.ld_dz, acc, lc, g, a.alpha, qv[0], qv[1]);
  atomicAdd(&tgk[tb_cur[0]], tg_cur[0]);
  atomicAdd(&tgk[tb_cur[1]], tg_cur[1]);
  __syncthreads();
  for (int e = tid; e < range; e += blockDim.x) {
    const float gsum = s_gpos[e];
    if (gsum != 0.0f) atomicAdd(&a.dpos[clampi(a.pos_center + e - 31, 0, a.pos_len - 1)], gsum);
  }
  if (tid < 64 && s_tgk[tid] != 0.0f) atomicAdd(&a.dtime[min(63 - tid, a.nb - 1)], s_tgk[tid]);
}

// dK and dV for the 32 key rows of one block and one head per wave.
template <int DH>
__global__ __launch_bounds__(512) void attn_train_kv_bf16_kernel(BwdAttnArgs a) {
  constexpr int NC = DH / 32, NCT = DH / 16;
  __shared__ float s_tvk[64];   // by time key + 32
  __shared__ float s_win[kMaxWaves][64];
  __shared__ int64_t s_ts[kMaxWaves][32];
  __shared__ uint32_t s_ts32[kMaxWaves][32];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kMaxWaves][32 * (DH + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t s_d[kMaxWaves][32 * (DH + 8)];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, g = lane >> 4;
  const Place pl = place(a, false, wave, nw);
  const int64_t s0 = a.offsets[pl.seq];
  const int L = static_cast<int>(a.offsets[pl.seq + 1] - s0);
  const int j0 = pl.blk * 32;
  if (j0 >= L) return;
  if (tid < 64) s_tvk[tid] = a.time_bias[min(63 - tid, a.nb - 1)];
  const float* tvk = s_tvk + 32;
  __syncthreads();

  const int d = a.d_model;
  const int64_t base = s0 * d + pl.h * DH;
  const uint16_t* Qs = a.q16 + base;
  const uint16_t* Ds = a.dav16 + base;
  const int64_t* Ts = a.ts + s0;
  uint16_t* qblk = s_q[wave];
  uint16_t* dblk = s_d[wave];
  bf16x8 kf[2][NC], vf[2][NC];
  bool kv[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int krow = min(j0 + 16 * kt + lc, L - 1);
    kv[kt] = j0 + 16 * kt + lc < L;
    load_row16<NC>(a.k16 + base + krow * d, g, kf[kt]);
    load_row16<NC>(a.v16 + base + krow * d, g, vf[kt]);
  }
  float* win = s_win[wave];
  int64_t* qts = s_ts[wave];
  uint32_t* qts32 = s_ts32[wave];
  // times as 32-bit offsets from the block's first key time where they fit
  const int64_t tref = Ts[j0];
  int64_t tk[2];
  uint32_t tk32[2];
  bool fk = true;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    tk[kt] = Ts[min(j0 + 16 * kt + lc, L - 1)];
    const uint64_t off = time_off(tk[kt], tref);
    fk = fk && time_fits32(off);
    tk32[kt] = static_cast<uint32_t>(off);
  }
  const bool fast_k = __builtin_amdgcn_ballot_w64(!fk) == 0;
  f32x4 dk[NCT][2], dv[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) dk[ct][0] = dk[ct][1] = dv[ct][0] = dv[ct][1] = f32x4{};
  const int nblk = (L + 31) >> 5;
  // window entry e <-> difference 32 qb - j0 - 31 + e; fetched a block ahead
  float wv = a.pos_bias[clampi(a.pos_center - 31 + lane, 0, a.pos_len - 1)];
  int64_t tsv = Ts[min(j0 + (lane & 31), L - 1)];
  // the block's Q and dAV rows; each step requests the next block's rows
  // into the same registers once the score products and the stashes have
  // read them
  bf16x8 qf[2][NC], df[2][NC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = min(j0 + 16 * qt + lc, L - 1);
    load_row16<NC>(Qs + qrow * d, g, qf[qt]);
    load_row16<NC>(Ds + qrow * d, g, df[qt]);
  }
  for (int qb = pl.blk; qb < nblk; ++qb) {
    const int q0 = qb * 32, D = q0 - j0;
    win[lane] = wv;
    const uint64_t qoff = time_off(tsv, tref);
    const bool fast = fast_k && __builtin_amdgcn_ballot_w64(!time_fits32(qoff)) == 0;
    if (lane < 32) {
      qts[lane] = tsv;
      qts32[lane] = static_cast<uint32_t>(qoff);
    }
    wv = a.pos_bias[clampi(a.pos_center + D + 1 + lane, 0, a.pos_len - 1)];
    tsv = Ts[min(q0 + 32 + (lane & 31), L - 1)];
    // S = Q K^T (rows: queries, columns: keys); dP = dAV V^T
    f32x4 sacc[2][2], pacc[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sacc[qt][kt] = pacc[qt][kt] = f32x4{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc[qt][kt] = mfma_16x16x32(qf[qt][c], kf[kt][c], sacc[qt][kt]);
          pacc[qt][kt] = mfma_16x16x32(df[qt][c], vf[kt][c], pacc[qt][kt]);
        }
      }
    // this block's queries and dAV rows, for the transposed reads
    stash_block<DH>(qblk, qf, lc, g);
    stash_block<DH>(dblk, df, lc, g);
    if (qb + 1 < nblk) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int qrow = min(q0 + 32 + 16 * qt + lc, L - 1);
        load_row16<NC>(Qs + qrow * d, g, qf[qt]);
        load_row16<NC>(Ds + qrow * d, g, df[qt]);
      }
    }
    // time buckets of the block's pairs, in 32 bits where the times allow
    int tbq[2][4][2];
    if (fast) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t tqr = qts32[16 * qt + 4 * g + r];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) tbq[qt][r][kt] = time_key32(tqr, tk32[kt]);
        }
    } else {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t tqr = qts[16 * qt + 4 * g + r];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) tbq[qt][r][kt] = time_key64(tqr - tk[kt]);
        }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ir = 16 * qt + 4 * g + r;   // query row in the block
        const bool qok = q0 + ir < L;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int jr = 16 * kt + lc;        // key row in the block
          const bool vis = kv[kt] && qok && (j0 + jr <= q0 + ir);
          const int tb = tbq[qt][r][kt];
          const float sc = a.alpha * sacc[qt][kt][r] + win[ir - jr + 31] + tvk[tb];
          const float sg = sigmoid_t(sc);
          sacc[qt][kt][r] = vis ? sc * sg : 0.0f;
          pacc[qt][kt][r] = vis ? pacc[qt][kt][r] * sg * (1.0f + sc * (1.0f - sg)) : 0.0f;
        }
      }
    // dV^T += dAV^T P and dK^T += Q^T dS over the block's 32 queries
    bf16x8 bp[2], bs[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bp[kt] = pack_slots(sacc[0][kt], sacc[1][kt]);
      bs[kt] = pack_slots(pacc[0][kt], pacc[1][kt]);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const bf16x8 dt_op = load_block_tr<DH>(dblk, ct, lc, g);
      const bf16x8 qt_op = load_block_tr<DH>(qblk, ct, lc, g);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        dv[ct][kt] = mfma_16x16x32(dt_op, bp[kt], dv[ct][kt]);
        dk[ct][kt] = mfma_16x16x32(qt_op, bs[kt], dk[ct][kt]);
      }
    }
  }
  store_tiles16<NCT>(a.dk + (s0 + j0) * a.ld_dz + pl.h * DH, a.ld_dz, dk, lc, g, a.alpha, kv[0], kv[1]);
  store_tiles16<NCT>(a.dv + (s0 + j0) * a.ld_dz + pl.h * DH, a.ld_dz, dv, lc, g, 1.0f, kv[0], kv[1]);
}

// AV for the 32 query rows of one block and one head per wave, from bf16
// Q, K and V on the bf16 matrix cores (plain causal attention, the layer's
// forward where no other bf16 kernel serves the head dimension): per 32-key
// block S^T = K Q^T, P = SiLU(S) masked, AV^T += V^T P^T. The bias, the
// 32-bit time keys and the operand layouts are those of the dQ kernel above,
// with V stashed for the transposed reads in place of K.
template <int DH>
__global__ __launch_bounds__(512) void attn_fwd_bf16_rows_kernel(BwdAttnArgs a) {
  constexpr int NC = DH / 32, NCT = DH / 16;
  __shared__ float s_tvk[64];   // by time key + 32
  __shared__ float s_win[kMaxWaves][64];
  __shared__ int64_t s_ts[kMaxWaves][32];
  __shared__ uint32_t s_ts32[kMaxWaves][32];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kMaxWaves][32 * (DH + 8)];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, g = lane >> 4;
  const Place pl = place(a, true, wave, nw);
  const int64_t s0 = a.offsets[pl.seq];
  const int L = static_cast<int>(a.offsets[pl.seq + 1] - s0);
  const int q0 = pl.blk * 32;
  if (q0 >= L) return;   // the whole workgroup: same sequence and block
  if (tid < 64) s_tvk[tid] = a.time_bias[min(63 - tid, a.nb - 1)];
  __syncthreads();

  const int d = a.d_model;
  const int64_t base = s0 * d + pl.h * DH;
  const uint16_t* Ks = a.k16 + base;
  const uint16_t* Vs = a.v16 + base;
  const int64_t* Ts = a.ts + s0;
  uint16_t* vblk = s_v[wave];
  bf16x8 qf[2][NC];
  int64_t tq[2];
  uint32_t tq32[2];
  bool qv[2];
  const int64_t tref = Ts[q0];
  bool fq = true;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = min(q0 + 16 * qt + lc, L - 1);
    qv[qt] = q0 + 16 * qt + lc < L;
    load_row16<NC>(a.q16 + base + qrow * d, g, qf[qt]);
    tq[qt] = Ts[qrow];
    const uint64_t off = time_off(tq[qt], tref);
    fq = fq && time_fits32(off);
    tq32[qt] = static_cast<uint32_t>(off);
  }
  const bool fast_q = __builtin_amdgcn_ballot_w64(!fq) == 0;
  float* win = s_win[wave];
  int64_t* kts = s_ts[wave];
  uint32_t* kts32 = s_ts32[wave];
  const float* tvk = s_tvk + 32;
  f32x4 acc[NCT][2];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct][0] = acc[ct][1] = f32x4{};
  float wv = a.pos_bias[clampi(a.pos_center + q0 - 31 + lane, 0, a.pos_len - 1)];
  int64_t tsv = Ts[min(lane & 31, L - 1)];
  // the block's K and V rows; the next block's go into the same registers
  // once the score products and the stash have read them
  bf16x8 kf[2][NC], vf[2][NC];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int krow = min(16 * kt + lc, L - 1);
    load_row16<NC>(Ks + krow * d, g, kf[kt]);
    load_row16<NC>(Vs + krow * d, g, vf[kt]);
  }

  for (int kb = 0; kb <= pl.blk; ++kb) {
    const int j0 = kb * 32, D = q0 - j0;
    win[lane] = wv;
    const uint64_t koff = time_off(tsv, tref);
    const bool fast = fast_q && __builtin_amdgcn_ballot_w64(!time_fits32(koff)) == 0;
    if (lane < 32) {
      kts[lane] = tsv;
      kts32[lane] = static_cast<uint32_t>(koff);
    }
    wv = a.pos_bias[clampi(a.pos_center + D - 63 + lane, 0, a.pos_len - 1)];
    tsv = Ts[min(j0 + 32 + (lane & 31), L - 1)];
    // S^T = K Q^T (rows: keys, columns: queries)
    f32x4 sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        sacc[kt][qt] = f32x4{};
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc[kt][qt] = mfma_16x16x32(kf[kt][c], qf[qt][c], sacc[kt][qt]);
      }
    // this block's values, for the transposed reads of the second product
    stash_block<DH>(vblk, vf, lc, g);
    if (kb < pl.blk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int krow = min(j0 + 32 + 16 * kt + lc, L - 1);
        load_row16<NC>(Ks + krow * d, g, kf[kt]);
        load_row16<NC>(Vs + krow * d, g, vf[kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float wq[4][2], tvq[4][2];
      int tbq[4][2];
      if (fast) {
        uint32_t tk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) tk[r] = kts32[16 * kt + 4 * g + r];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) tbq[r][qt] = time_key32(tq32[qt], tk[r]);
      } else {
        int64_t tk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) tk[r] = kts[16 * kt + 4 * g + r];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) tbq[r][qt] = time_key64(tq[qt] - tk[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) wq[r][qt] = win[16 * qt + lc - (16 * kt + 4 * g + r) + 31];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) tvq[r][qt] = tvk[tbq[r][qt]];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jr = 16 * kt + 4 * g + r;   // key row in the block
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int ir = 16 * qt + lc;        // query row in the block
          const bool vis = qv[qt] && (j0 + jr <= q0 + ir);
          const float sc = a.alpha * sacc[kt][qt][r] + wq[r][qt] + tvq[r][qt];
          const float pv = sc * sigmoid_t(sc);
          sacc[kt][qt][r] = vis ? pv : 0.0f;
        }
      }
    }
    // AV^T += V^T P^T over the block's 32 keys
    bf16x8 bp[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) bp[qt] = pack_slots(sacc[0][qt], sacc[1][qt]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const bf16x8 vt_op = load_block_tr<DH>(vblk, ct, lc, g);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) acc[ct][qt] = mfma_16x16x32(vt_op, bp[qt], acc[ct][qt]);
    }
  }
  store_tiles16<NCT>(a.av + (s0 + q0) * a.d_model + pl.h * DH, a.d_model, acc, lc, g, 1.0f, qv[0], qv[1]);
}

// fp32 -> bf16 (round to nearest even), n a multiple of 4.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float4* __restrict__ src, uint2* __restrict__ dst,
                                                      int64_t n4) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const float4 v = src[i];
    dst[i] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

// Waves per workgroup: the largest divisor of num_heads up to kMaxWaves.
int waves_for(int num_heads) {
  for (int w = kMaxWaves; w > 1; --w)
    if (num_heads % w == 0) return w;
  return 1;
}

template <typename K>
hipError_t launch_train(K kernel, const BwdAttnArgs& a, hipStream_t s) {
  const int nw = waves_for(a.num_heads);
  const int64_t nblk = (static_cast<int64_t>(a.max_seq_len) + 31) / 32;
  const int64_t grid = nblk * a.num_seqs * (a.num_heads / nw);
  if (grid == 0) return hipSuccess;
  // row offsets inside one sequence are int32
  if (static_cast<int64_t>(a.max_seq_len) * a.d_model >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(64 * nw), 0, s, a);
  return hipGetLastError();
}

}  // namespace


hipError_t launch_attn_train_fwd(const BwdAttnArgs& a, hipStream_t s) {
  return a.head_dim == 32 ? launch_train(attn_train_q_kernel<32, true>, a, s)
                          : launch_train(attn_train_q_kernel<64, true>, a, s);
}

hipError_t launch_attn_bwd_bf16(const BwdAttnArgs& a, hipStream_t s) {
  if (!a.q16 || !a.k16 || !a.v16 || !a.dav16) return hipErrorInvalidValue;
  const bool lng = static_cast<int64_t>(a.max_seq_len) + 64 > kPosCapB;
  hipError_t e;
  if (a.head_dim == 32)
    e = lng ? launch_train(attn_train_dq_bf16_kernel<32, true>, a, s)
            : launch_train(attn_train_dq_bf16_kernel<32, false>, a, s);
  else
    e = lng ? launch_train(attn_train_dq_bf16_kernel<64, true>, a, s)
            : launch_train(attn_train_dq_bf16_kernel<64, false>, a, s);
  if (e != hipSuccess) return e;
  return a.head_dim == 32 ? launch_train(attn_train_kv_bf16_kernel<32>, a, s)
                          : launch_train(attn_train_kv_bf16_kernel<64>, a, s);
}

hipError_t launch_attn_fwd_bf16_rows(const BwdAttnArgs& a, hipStream_t s) {
  if (!a.q16 || !a.k16 || !a.v16 || !a.av) return hipErrorInvalidValue;
  return a.head_dim == 32 ? launch_train(attn_fwd_bf16_rows_kernel<32>, a, s)
                          : launch_train(attn_fwd_bf16_rows_kernel<64>, a, s);
}

hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(src), reinterpret_cast<uint2*>(dst), n4);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const BwdAttnArgs& a, hipStream_t s) {
  const bool lng = static_cast<int64_t>(a.max_seq_len) + 64 > kPosCap;
  hipError_t e;
  if (a.head_dim == 32)
    e = lng ? launch_train(attn_train_q_kernel<32, false, true>, a, s)
            : launch_train(attn_train_q_kernel<32, false, false>, a, s);
  else
    e = lng ? launch_train(attn_train_q_kernel<64, false, true>, a, s)
            : launch_train(attn_train_q_kernel<64, false, false>, a, s);
  if (e != hipSuccess) return e;
  return a.head_dim == 32 ? launch_train(attn_train_kv_kernel<32>, a, s)
                          : launch_train(attn_train_kv_kernel<64>, a, s);
}

}  // namespace hstu
