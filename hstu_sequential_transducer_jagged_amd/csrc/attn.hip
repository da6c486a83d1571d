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
// bf16 kernel (head_dim 64) design:
//  * a workgroup owns one 64-query tile of one sequence for HPB heads, one
//    wave per head, and walks the visible 32-key tiles (tiles above the
//    diagonal and tiles of other targets are never visited);
//  * K and V tiles of all HPB heads arrive by direct global->LDS loads
//    (global_load_lds_dwordx4) into a double buffer, one tile ahead;
//  * the relative bias is shared by all heads: the workgroup builds each
//    64 x 32 bias tile once, one step ahead, from per-key timestamps staged in
//    LDS and a sliding window of the position table, and every wave uses it
//    as the initial accumulator of its Q.K MFMAs (the add is free);
//  * scores are produced directly in the base-2 domain: Q is prescaled by
//    -alpha*log2(e) and the bias by -log2(e), so with S' = -log2(e) S
//    SiLU(S) = -ln2 * S' / (1 + 2^S'): one exp2, one add, one rcp and one
//    mul per score; -ln2 is applied once to the output; invisible pairs get
//    a bias that sends 2^S' to +inf (P = 0);
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator layout of S^T
//    (lane = query, 16 keys) is the A-operand layout of the S.V MFMA, so P
//    stays in registers; V's B operand is read with ds_read_b64_tr_b16
//    (transposing 16-bit reads) from the row-major tile;
//  * software pipeline in half tiles: while the score MFMAs of one 32-query
//    block run, the SiLU and P.V of the previous block do, so the matrix
//    cores and the vector ALUs of a wave overlap; the DMA of the next tile
//    is spread over the step;
//  * time buckets are exact integers: 32-bit |dt|+1 and a leading-zero count
//    when every pair of the tile is within 2^30 s of the block's reference
//    time, a 64-bit path otherwise.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace hstu {
namespace {

constexpr int kBM = 64;   // query rows per workgroup
constexpr int kBN = 32;   // keys per step
constexpr int kDH = 64;   // head dim of the bf16 kernel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaskBias = 1.0e30f;   // base-2 score bias of an invisible pair
constexpr int kPosWin = 128;           // position-window entries per tile

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

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

// Per-key data of one key tile, delivered to LDS by DMA two tiles ahead.
struct KeyData {
  alignas(16) uint32_t tlo[kBN];    // low words of the key timestamps
  alignas(16) uint32_t thi[kBN];    // high words (64-bit path)
  alignas(16) float pos[kPosWin];   // raw position-bias window, entry e <-> dp = w0 + e
};

// Bytes per staged K / V row of HPB heads. The pads put the rows of one MFMA
// operand read on distinct LDS banks: 16 B for the 16-lane b128 reads of K,
// 64 B for the 32-lane transposing b64 reads of V.
template <int HPB>
struct Rows {
  static constexpr int ROWBK = HPB * kDH * 2 + 16;
  static constexpr int ROWBV = HPB * kDH * 2 + 64;
};

// Position of key kk (block key index: cache rows first).
__device__ __forceinline__ int key_pos(int kk, int nc, int first_tgt) {
  return kk < nc ? kk : nc + min(kk - nc, first_tgt);
}

// Block-uniform integers of one query tile.
struct Ctx {
  int64_t s, cs;
  int L, nc, first_tgt, q0, q_hi, nkeys, d, col0, pmin_q, pos_len, pos_center;
  int no_self;        // targets do not see themselves
  uint32_t tb_lo;     // low word of the block's reference time (minimum timestamp)
  int wide;           // the block's timestamps span >= 2^31 s: 64-bit bucket path
};

// Window origin (position difference of window entry 0) of key tile `tile`.
__device__ __forceinline__ int window_origin(const Ctx& c, int tile) {
  const int klast = min(tile * kBN + kBN, c.nkeys) - 1;
  return c.pmin_q - key_pos(klast, c.nc, c.first_tgt);
}

// Source row (global element offset of the row start) of block key kk.
__device__ __forceinline__ int64_t key_row(const Ctx& c, int kk) {
  return kk < c.nc ? (c.cs + kk) : (c.s + kk - c.nc);
}

// DMA of a tile's key data: wave 0 the timestamps (lanes 0..31 low words,
// 32..63 high words), waves 1 and 2 the two halves of the position window.
template <int HPB>
__device__ __forceinline__ void load_keydata(const Ctx& c, const int64_t* ts, const int64_t* c_ts,
                                             const float* pos_bias, KeyData& kd, int tile, int wave,
                                             int lane) {
  if (wave == 0) {
    const int kk = min(tile * kBN + (lane & (kBN - 1)), c.nkeys - 1);
    const int64_t* tp = kk < c.nc ? c_ts + (c.cs + kk) : ts + (c.s + kk - c.nc);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tp) + (lane >> 5);
    __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, kd.tlo), 4, 0, 0);
  } else if (wave <= 2 || HPB < 4) {
    // with fewer than 3 waves, wave 0 / 1 issue the window halves too
    const int w0 = window_origin(c, tile);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (HPB >= 4 && half != wave - 1) continue;
      int idx = c.pos_center + w0 + half * 64 + lane;
      idx = idx < 0 ? 0 : (idx >= c.pos_len ? c.pos_len - 1 : idx);
      __builtin_amdgcn_global_load_lds(pos_bias + idx, LDS_PTR(void, kd.pos + half * 64), 4, 0, 0);
    }
  }
  if (HPB < 4 && wave == 0) {
    const int w0 = window_origin(c, tile);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      int idx = c.pos_center + w0 + half * 64 + lane;
      idx = idx < 0 ? 0 : (idx >= c.pos_len ? c.pos_len - 1 : idx);
      __builtin_amdgcn_global_load_lds(pos_bias + idx, LDS_PTR(void, kd.pos + half * 64), 4, 0, 0);
    }
  }
}

// One DMA row of a K or V tile: block key min(k0 + r, nkeys - 1) into LDS row
// r. The source row is wave-uniform (scalar address arithmetic); the lane adds
// its 16-byte column offset.
template <int HPB, int ROWB>
__device__ __forceinline__ void dma_row(const Ctx& c, const uint16_t* base_o, const uint16_t* base_c,
                                        uint8_t* dst, int k0, int r, int lane) {
  if (HPB < 8 && lane >= HPB * 8) return;
  const int kk = min(k0 + r, c.nkeys - 1);
  const uint16_t* src = (kk < c.nc ? base_c : base_o) + static_cast<int64_t>(kk) * c.d;
  __builtin_amdgcn_global_load_lds(src + lane * 8, LDS_PTR(void, dst + r * ROWB), 16, 0, 0);
}

// P = S' / (1 + 2^S') for scores [8h, 8h + 8) of one accumulator, packed to
// bf16 as one A operand of the P.V MFMA.
__device__ __forceinline__ bf16x8 silu8(const f32x16& st, int h) {
  uint32_t pk[4];
#pragma unroll
  for (int r = 0; r < 8; r += 2) {
    const float x0 = st[8 * h + r], x1 = st[8 * h + r + 1];
    const float p0 = x0 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x0));
    const float p1 = x1 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x1));
    pk[r >> 1] = pack_bf16x2(p0, p1);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
}

// P for scores [4q, 4q + 4) of one accumulator, as two packed bf16 pairs.
__device__ __forceinline__ void silu4(const f32x16& st, int q, uint32_t& w0, uint32_t& w1) {
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x = st[4 * q + r];
    p[r] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
  }
  w0 = pack_bf16x2(p[0], p[1]);
  w1 = pack_bf16x2(p[2], p[3]);
}

// One quarter (4 scores per lane) of load_bias_block.
__device__ __forceinline__ void load_bias_quarter(const float* bias, int qb, int j, int lane, f32x16& st) {
  const float4 bv = *reinterpret_cast<const float4*>(&bias[((qb * 4 + j) * 64 + lane) * 4]);
  st[4 * j + 0] = bv.x;
  st[4 * j + 1] = bv.y;
  st[4 * j + 2] = bv.z;
  st[4 * j + 3] = bv.w;
}

// V operands of one 16-key half (both 32-dim blocks).
template <int ROWB>
__device__ __forceinline__ void load_v_half(const uint8_t* vb, int voff, int kh, bf16x8 (&vf)[2][2]) {
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const uint8_t* p = vb + voff + kh * 16 * ROWB + db * 64;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * ROWB));
    vf[db][kh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// Bias tile rows of one 32-query block as the initial S^T accumulator.
__device__ __forceinline__ void load_bias_block(const float* bias, int qb, int lane, f32x16& st) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 bv = *reinterpret_cast<const float4*>(&bias[((qb * 4 + j) * 64 + lane) * 4]);
    st[4 * j + 0] = bv.x;
    st[4 * j + 1] = bv.y;
    st[4 * j + 2] = bv.z;
    st[4 * j + 3] = bv.w;
  }
}

// Per-thread slot data of the bias builder: slot = (qb*4 + j)*64 + l covers
// query qb*32 + l%32 and keys 8j + 4(l/32) + r, r = 0..3 (the S^T
// accumulator order of v_mfma_f32_32x32x16).
template <int SPT>
struct SlotQ {
  int qi[SPT], pq[SPT];
  uint32_t uq[SPT];     // query time relative to the block reference (32-bit path)
  int64_t tq[SPT];      // raw query time (64-bit path)
};

// Bias tile (base-2 domain) of key tile `tile` from its key data.
template <int HPB>
__device__ __forceinline__ void build_bias(const Ctx& c, const SlotQ<512 / (64 * HPB)>& sq,
                                           const KeyData& kd, float* bias, const float* tb_clz,
                                           const float* tb_lin, int nb, int tile, int tid) {
  constexpr int NT = 64 * HPB;
  constexpr int SPT = 512 / NT;
  const int k0 = tile * kBN;
  const int w0 = window_origin(c, tile);
  // all keys are non-targets visible to every query of the block
  const bool full = (k0 + kBN - 1 - c.nc <= c.q0) && (k0 + kBN - 1 - c.nc < c.first_tgt);
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int slot = tid + i * NT;
    const int kr = 8 * ((slot >> 6) & 3) + 4 * ((slot >> 5) & 1);
    const int kbase = k0 + kr;
    const int qi = sq.qi[i];
    float b[4];
    if (full && !c.wide) {
      const uint4 t4 = *reinterpret_cast<const uint4*>(&kd.tlo[kr]);
      const uint32_t tk[4] = {t4.x, t4.y, t4.z, t4.w};
      const float* pw = kd.pos + (sq.pq[i] - kbase - w0);   // p_k = kk for non-target keys
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t x = sq.uq[i], y = tk[r] - c.tb_lo;
        const uint32_t ad = (x > y ? x - y : y - x) + 1u;   // |dt| + 1 >= 1
        b[r] = __builtin_fmaf(pw[-r], -kLog2e, tb_clz[__builtin_clz(ad)]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kbase + r;
        const int jo = kk - c.nc;
        const bool vis = qi < c.L && kk < c.nkeys &&
                         (kk < c.nc ||
                          (jo <= qi && (jo < c.first_tgt || (jo == qi && !(c.no_self && qi >= c.first_tgt)))));
        int pidx = sq.pq[i] - key_pos(kk, c.nc, c.first_tgt) - w0;
        pidx = pidx < 0 ? 0 : (pidx >= kPosWin ? kPosWin - 1 : pidx);
        float tbv;
        if (!c.wide) {
          const uint32_t x = sq.uq[i], y = kd.tlo[kr + r] - c.tb_lo;
          const uint32_t ad = (x > y ? x - y : y - x) + 1u;
          tbv = tb_clz[__builtin_clz(ad)];
        } else {
          const int64_t tk = static_cast<int64_t>((static_cast<uint64_t>(kd.thi[kr + r]) << 32) |
                                                  kd.tlo[kr + r]);
          tbv = tb_lin[time_bucket64(sq.tq[i] - tk, nb)];
        }
        b[r] = vis ? __builtin_fmaf(kd.pos[pidx], -kLog2e, tbv) : kMaskBias;
      }
    }
    *reinterpret_cast<float4*>(&bias[slot * 4]) = make_float4(b[0], b[1], b[2], b[3]);
  }
}

// The full-tile bias of build_bias split in three pieces, so that its LDS
// round trips overlap other work: issue the key-data reads, then (once they
// are back) the time-bias lookups, then combine and store. Valid for tiles
// whose keys are all visible non-targets and a 32-bit time span; on other
// tiles it writes bounded garbage that build_bias then overwrites.
template <int SPT>
struct FastBias {
  uint32_t tk[SPT][4];
  float pw[SPT][4];
  float tb[SPT][4];
};

template <int HPB>
__device__ __forceinline__ void fast_bias_issue(const Ctx& c, const SlotQ<512 / (64 * HPB)>& sq,
                                                const KeyData& kd, int tile, int tid,
                                                FastBias<512 / (64 * HPB)>& fb) {
  constexpr int NT = 64 * HPB;
  constexpr int SPT = 512 / NT;
  const int k0 = tile * kBN;
  const int w0 = window_origin(c, tile);
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int slot = tid + i * NT;
    const int kr = 8 * ((slot >> 6) & 3) + 4 * ((slot >> 5) & 1);
    const uint4 t4 = *reinterpret_cast<const uint4*>(&kd.tlo[kr]);
    fb.tk[i][0] = t4.x;
    fb.tk[i][1] = t4.y;
    fb.tk[i][2] = t4.z;
    fb.tk[i][3] = t4.w;
    int pb = sq.pq[i] - (k0 + kr) - w0;   // p_k = kk for non-target keys
    pb = pb < 3 ? 3 : (pb > kPosWin - 1 ? kPosWin - 1 : pb);
#pragma unroll
    for (int r = 0; r < 4; ++r) fb.pw[i][r] = kd.pos[pb - r];
  }
}

template <int HPB>
__device__ __forceinline__ void fast_bias_lookup(const Ctx& c, const SlotQ<512 / (64 * HPB)>& sq,
                                                 const float* tb_clz, FastBias<512 / (64 * HPB)>& fb) {
  constexpr int SPT = 512 / (64 * HPB);
#pragma unroll
  for (int i = 0; i < SPT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t x = sq.uq[i], y = fb.tk[i][r] - c.tb_lo;
      const uint32_t ad = (x > y ? x - y : y - x) + 1u;   // |dt| + 1 >= 1
      fb.tb[i][r] = tb_clz[__builtin_clz(ad)];
    }
}

template <int HPB>
__device__ __forceinline__ void fast_bias_store(const FastBias<512 / (64 * HPB)>& fb, float* bias, int tid) {
  constexpr int NT = 64 * HPB;
  constexpr int SPT = 512 / NT;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int slot = tid + i * NT;
    float b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // pins the combine here: computed earlier, it would make the wave
      // wait for every LDS read in flight
      float tb = fb.tb[i][r];
      asm volatile("" : "+v"(tb));
      b[r] = __builtin_fmaf(fb.pw[i][r], -kLog2e, tb);
    }
    *reinterpret_cast<float4*>(&bias[slot * 4]) = make_float4(b[0], b[1], b[2], b[3]);
  }
}

// DMA slot `slot` (0..7) of a step: an eighth of the K and V rows of key
// tile k0 / kBN (K rows in even slots, V rows in odd ones).
template <int HPB>
__device__ __forceinline__ void dma_slot(const Ctx& c, const uint16_t* kbase_o, const uint16_t* kbase_c,
                                         const uint16_t* vbase_o, const uint16_t* vbase_c,
                                         uint8_t* __restrict__ nk, uint8_t* __restrict__ nv, int k0, int slot,
                                         int wave, int lane) {
  constexpr int RPW = kBN / HPB;   // rows per wave of one tile
  constexpr int RPS = RPW / 4;     // rows per slot
#pragma unroll
  for (int it = 0; it < RPS; ++it) {
    const int r = wave + ((slot >> 1) * RPS + it) * HPB;
    if (slot & 1) dma_row<HPB, Rows<HPB>::ROWBV>(c, vbase_o, vbase_c, nv, k0, r, lane);
    else dma_row<HPB, Rows<HPB>::ROWBK>(c, kbase_o, kbase_c, nk, k0, r, lane);
  }
}

// One key step of the software pipeline (see the kernel). The LDS buffers
// are distinct restrict-qualified arguments: the compiler can then tell that
// a DMA into the next buffers does not alias the reads of the current ones,
// and issues the DMA early without making those reads wait for it. MORE: a
// later tile of the chunk follows (its DMA, key data and bias).
template <int HPB, bool MORE>
__device__ __forceinline__ void attn_step(
    const Ctx& c, const SlotQ<512 / (64 * HPB)>& sq, const AttnArgs& a, int st, int st_hi, int skip_a,
    int n_skip, const uint8_t* __restrict__ curK, const float* __restrict__ curB,
    const uint8_t* __restrict__ curV, uint8_t* __restrict__ nxtK, uint8_t* __restrict__ nxtV,
    float* __restrict__ nxtB, const KeyData* __restrict__ nxtD, KeyData* __restrict__ curD,
    const float* __restrict__ tb_clz, const float* __restrict__ tb_lin, const uint16_t* kbase_o,
    const uint16_t* kbase_c, const uint16_t* vbase_o, const uint16_t* vbase_c, const bf16x8 (&qf)[2][4],
    f32x16 (&acc)[2][2], f32x16& s0, f32x16& s1, bf16x8 (&vf)[2][2], int koff, int voff, int wave, int lane,
    int tid) {
  constexpr int ROWBV = Rows<HPB>::ROWBV;
  const int t1 = MORE ? (st + 1 < skip_a ? st + 1 : st + 1 + n_skip) : 0;
  const int k1 = t1 * kBN;
  // the bias of tile st+1 takes the split fast path when all its keys are
  // visible non-targets for the whole block and times fit 32 bits
  const bool fast1 = (k1 + kBN - 1 - c.nc <= c.q0) && (k1 + kBN - 1 - c.nc < c.first_tgt) && !c.wide;
  FastBias<512 / (64 * HPB)> fb;
  // A0: the key-data reads of tile st+1's bias go first, so that their
  // dependent time-bias lookups are not queued behind this step's big LDS
  // reads; DMA of the key data of tile st+2 and a quarter of the K/V rows
  if (MORE) fast_bias_issue<HPB>(c, sq, *nxtD, t1, tid, fb);
  if (MORE && st + 2 < st_hi) {
    const int t2 = st + 2 < skip_a ? st + 2 : st + 2 + n_skip;
    load_keydata<HPB>(c, a.ts, a.c_ts, a.pos_bias, *curD, t2, wave, lane);
  }
  if (MORE) {
    dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, nxtK, nxtV, k1, 0, wave, lane);
    dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, nxtK, nxtV, k1, 1, wave, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  // R0: SiLU of block 1 of tile st-1 in quarters, each quarter's registers
  // then refilled with the block-1 bias of tile st; P.V with V of tile
  // st-1, each half of vf then refilled with V of tile st; the score MFMAs
  // of block 0 in the second half; the rest of the DMA
  bf16x8 kf[4];
  {
    uint32_t w[8];
    silu4(s1, 0, w[0], w[1]);
    if (MORE) fast_bias_lookup<HPB>(c, sq, tb_clz, fb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      kf[cc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(curK + koff + cc * 32));
    load_bias_block(curB, 0, lane, s0);
    load_bias_quarter(curB, 1, 0, lane, s1);
    if (MORE) {
      dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, nxtK, nxtV, k1, 2, wave, lane);
      dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, nxtK, nxtV, k1, 3, wave, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sr = 1; sr < 4; ++sr) {
      silu4(s1, sr, w[2 * sr], w[2 * sr + 1]);
      load_bias_quarter(curB, 1, sr, lane, s1);
      if (MORE && sr < 3) {
        dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, nxtK, nxtV, k1, 2 + 2 * sr, wave, lane);
        dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, nxtK, nxtV, k1, 3 + 2 * sr, wave, lane);
      }
      if (sr >= 2) {
        s0 = mfma32(kf[2 * (sr - 2)], qf[0][2 * (sr - 2)], s0);
        s0 = mfma32(kf[2 * (sr - 2) + 1], qf[0][2 * (sr - 2) + 1], s0);
      }
      // the store waits for every LDS read issued before it (the DMA keeps
      // the compiler from counting partially): after the score MFMAs, which
      // wait for K and the bias anyway
      if (MORE && sr == 2) fast_bias_store<HPB>(fb, nxtB, tid);
      if (sr & 1) {
        const int kh = sr >> 1;
        const bf16x8 pk = __builtin_bit_cast(bf16x8, make_uint4(w[4 * kh], w[4 * kh + 1], w[4 * kh + 2], w[4 * kh + 3]));
#pragma unroll
        for (int db = 0; db < 2; ++db) acc[1][db] = mfma32(pk, vf[db][kh], acc[1][db]);
        load_v_half<ROWBV>(curV, voff, kh, vf);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // R1: SiLU of block 0 of tile st and its P.V; the score MFMAs of block 1
  {
    uint32_t w[8];
#pragma unroll
    for (int sr = 0; sr < 4; ++sr) {
      silu4(s0, sr, w[2 * sr], w[2 * sr + 1]);
      // two score MFMAs every other quarter: the block-1 bias read last in
      // R0 has time to land
      if (sr & 1) {
        s1 = mfma32(kf[sr - 1], qf[1][sr - 1], s1);
        s1 = mfma32(kf[sr], qf[1][sr], s1);
        const int kh = sr >> 1;
        const bf16x8 pk = __builtin_bit_cast(bf16x8, make_uint4(w[4 * kh], w[4 * kh + 1], w[4 * kh + 2], w[4 * kh + 3]));
#pragma unroll
        for (int db = 0; db < 2; ++db) acc[0][db] = mfma32(pk, vf[db][kh], acc[0][db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // keep the wait and the barrier after the SiLU of this step
    asm volatile("" ::"v"(w[7]));
  }
  // tiles off the fast path: the full bias builder overwrites the tile
  if (MORE && !fast1) build_bias<HPB>(c, sq, *nxtD, nxtB, tb_clz, tb_lin, a.nb, t1, tid);
  if (MORE) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// Number of key steps (32-key tiles visited) of query tile qt of a sequence:
// the cost the schedule sorts by.
__device__ __forceinline__ int tile_steps(const SeqInfo& si, int qt) {
  const int q0 = qt * kBM;
  const int q_hi = min(q0 + kBM, si.L);
  const int nkeys = si.nc + q_hi;
  const int n_kt = (nkeys + kBN - 1) / kBN;
  const int first_tgt = si.L - si.m;
  const int skip_a = (si.nc + first_tgt + kBN - 1) / kBN;
  const int skip_b = max((si.nc + q0) / kBN, skip_a);
  return n_kt - (skip_b - skip_a);
}

constexpr int kNumXcd = 8;            // XCDs of the chip; workgroup id -> XCD id % 8
constexpr int kCostBuckets = 1024;    // cost classes of the per-XCD sort
constexpr int kSchedHead = kNumXcd + 1;
constexpr int64_t kSplitMinUnits = 512;  // below this many items, key ranges are split
constexpr int kMaxSplits = 8;

// Key steps [lo, hi) of chunk c of an item with n steps: chunks of ceil(n / S)
// steps; trailing chunks may be empty.
__device__ __forceinline__ void chunk_range(int n, int S, int c, int& lo, int& hi) {
  const int per = (n + S - 1) / S;
  lo = min(c * per, n);
  hi = min(lo + per, n);
}

// Cost of work unit u = item * S + chunk: its key steps, at least 1 for a
// non-empty item (an empty chunk still writes its zero partial); 0 for an
// empty tile (never scheduled).
__device__ __forceinline__ int unit_cost(const AttnArgs& a, int n_qt, int u) {
  const int S = a.splits;
  const int i = u / S, ch = u - i * S;
  const int b = i / n_qt, t = i - b * n_qt;
  const SeqInfo si = seq_info(a, b);
  // tiles past max_seq_len (a violated contract) are never reached: t < n_qt
  if (t * kBM >= si.L) return 0;
  int lo, hi;
  chunk_range(tile_steps(si, t), S, ch, lo, hi);
  return max(hi - lo, 1);
}

// Work list of the bf16 attention. Items are the non-empty (sequence,
// 64-query tile) pairs, each cut into a.splits units of consecutive key steps
// (one unit per item unless the batch has few items); a unit's cost is its
// number of key steps.
//  1. Units, in (sequence, tile, chunk) order, are cut into kNumXcd contiguous runs
//     of equal total cost; run x goes to XCD x. The workgroups of one XCD
//     then work on one or a few sequences at a time and share their K/V rows
//     in that XCD's L2.
//  2. Within a run, items are counting-sorted by cost, most expensive first,
//     so that the XCD's compute units finish together.
// sched[x] (x = 0..8): first list index of XCD x (sched[8] = unit count);
// sched[9 + k]: unit ((seq * n_qt + tile) * splits + chunk) at list index k.
// Exclusive prefix sum over the 1024 threads of the block (wave scans by
// shuffles, then one pass over the 16 wave totals); *total receives the sum.
__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* wsum, long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long t = __shfl_up(inc, off, 64);
    if (lane >= off) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    long long w = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const long long t = __shfl_up(w, off, 64);
      if (lane >= off) w += t;
    }
    if (lane < 16) wsum[lane] = w;
  }
  __syncthreads();
  const long long excl = inc - v + (wave ? wsum[wave - 1] : 0);
  *total = wsum[15];
  __syncthreads();   // wsum may be reused by the next scan
  return excl;
}

__global__ __launch_bounds__(1024) void attn_schedule_kernel(AttnArgs a, int n_qt) {
  constexpr int kKeep = 8;   // unit costs per thread kept in registers between the passes
  __shared__ int cnt[kNumXcd * kCostBuckets];
  __shared__ long long wsum[16];
  const int tid = threadIdx.x;
  const int items = a.num_seqs * n_qt * a.splits;
  for (int i = tid; i < kNumXcd * kCostBuckets; i += 1024) cnt[i] = 0;
  // each thread owns a contiguous chunk of items
  const int per = (items + 1023) / 1024;
  const int i0 = min(tid * per, items), i1 = min(i0 + per, items);
  int cst[kKeep];
  long long sum = 0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    cst[k] = i0 + k < i1 ? unit_cost(a, n_qt, i0 + k) : 0;
    sum += cst[k];
  }
  for (int i = i0 + kKeep; i < i1; ++i) sum += unit_cost(a, n_qt, i);
  long long total_cost;
  const long long run0 = block_exclusive_scan(sum, wsum, &total_cost);   // also orders cnt's zeroing
  // sort key: XCD-major, cost descending; the item's XCD is the run holding
  // the midpoint of its cost interval
  auto key_of = [&](long long run, int c) __attribute__((always_inline)) {
    const int x = static_cast<int>(min(static_cast<long long>(kNumXcd - 1),
                                       ((2 * run + c) * kNumXcd) / (2 * total_cost)));
    return x * kCostBuckets + (kCostBuckets - 1 - min(c, kCostBuckets - 1));
  };
  long long run = run0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    if (cst[k] > 0) atomicAdd(&cnt[key_of(run, cst[k])], 1);
    run += cst[k];
  }
  for (int i = i0 + kKeep; i < i1; ++i) {
    const int c = unit_cost(a, n_qt, i);
    if (c > 0) atomicAdd(&cnt[key_of(run, c)], 1);
    run += c;
  }
  __syncthreads();
  // exclusive scan of the kNumXcd * kCostBuckets counters, 8 per thread
  constexpr int kPer = kNumXcd * kCostBuckets / 1024;
  int loc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) loc += cnt[tid * kPer + i];
  long long units;
  int base = static_cast<int>(block_exclusive_scan(loc, wsum, &units));
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = cnt[tid * kPer + i];
    cnt[tid * kPer + i] = base;
    base += c;
  }
  __syncthreads();
  if (tid < kNumXcd) a.sched[tid] = cnt[tid * kCostBuckets];
  if (tid == kNumXcd) a.sched[kNumXcd] = static_cast<int>(units);
  run = run0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    if (cst[k] > 0) a.sched[kSchedHead + atomicAdd(&cnt[key_of(run, cst[k])], 1)] = i0 + k;
    run += cst[k];
  }
  for (int i = i0 + kKeep; i < i1; ++i) {
    const int c = unit_cost(a, n_qt, i);
    if (c > 0) a.sched[kSchedHead + atomicAdd(&cnt[key_of(run, c)], 1)] = i;
    run += c;
  }
}

template <int HPB, bool FUSE_NG>
__global__ __launch_bounds__(64 * HPB, 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = 64 * HPB;
  constexpr int ROWBK = Rows<HPB>::ROWBK;
  constexpr int ROWBV = Rows<HPB>::ROWBV;
  constexpr int SPT = 512 / NT;   // bias slots per thread (512 slots of 4 pairs)
  // K and V double buffers in one block: after the last step it holds the
  // fp32 output tile of the fused norm_gate epilogue (64 x d floats fit:
  // 64 * HPB * 256 bytes against 64 * (HPB * 256 + 80)). The steps receive
  // the buffers as distinct restrict-qualified pointers, so a DMA into one
  // does not make the compiler wait before reads of another.
  __shared__ __attribute__((aligned(16))) uint8_t skv[2 * kBN * ROWBK + 2 * kBN * ROWBV];
  uint8_t* const sK0 = skv;
  uint8_t* const sK1 = skv + kBN * ROWBK;
  uint8_t* const sV0 = skv + 2 * kBN * ROWBK;
  uint8_t* const sV1 = sV0 + kBN * ROWBV;
  __shared__ __attribute__((aligned(16))) float sB0[kBM * kBN];
  __shared__ __attribute__((aligned(16))) float sB1[kBM * kBN];
  __shared__ KeyData sD0, sD1;
  __shared__ float tb_clz[32];   // base-2 time bias indexed by clz(|dt|+1)
  __shared__ float tb_lin[64];   // base-2 time bias indexed by bucket
  __shared__ int64_t red_min[HPB], red_max[HPB];

  // Work items of this workgroup: workgroup g runs on XCD g % 8 and takes
  // that XCD's list entries g / 8, g / 8 + gridDim.x / 8, ...
  const int xcd = blockIdx.x % kNumXcd;
  const int list_end = a.sched[xcd + 1];
  const int list_step = gridDim.x / kNumXcd;
  for (int li = a.sched[xcd] + static_cast<int>(blockIdx.x) / kNumXcd; li < list_end; li += list_step) {
  __syncthreads();   // the previous item's LDS reads are done
  const int unit = a.sched[kSchedHead + li];
  const int item = unit / a.splits;
  const int chunk = unit - item * a.splits;
  const int n_qt = (a.max_seq_len + kBM - 1) / kBM;
  const int seq = item / n_qt;
  const int qt = item - seq * n_qt;
  const SeqInfo si = seq_info(a, seq);
  const int q0 = qt * kBM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int hcol = wave * kDH;                     // this wave's head within the group

  Ctx c;
  c.s = si.s;
  c.cs = si.cs;
  c.L = si.L;
  c.nc = si.nc;
  c.first_tgt = si.L - si.m;
  c.no_self = a.no_self;
  c.q0 = q0;
  c.q_hi = min(q0 + kBM, si.L);
  c.nkeys = c.nc + c.q_hi;
  c.d = a.d_model;
  c.col0 = blockIdx.y * HPB * kDH;
  c.pmin_q = c.nc + min(q0, c.first_tgt);
  c.pos_len = a.pos_len;
  c.pos_center = a.pos_center;

  // ---- reference time: min / max timestamp over every key of the block
  // (queries are among them) ----
  {
    int64_t tmin = INT64_MAX, tmax = INT64_MIN;
    for (int kk = tid; kk < c.nkeys; kk += NT) {
      const int64_t t = kk < c.nc ? a.c_ts[c.cs + kk] : a.ts[c.s + kk - c.nc];
      tmin = min(tmin, t);
      tmax = max(tmax, t);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      tmin = min(tmin, static_cast<int64_t>(__shfl_xor(tmin, off, 64)));
      tmax = max(tmax, static_cast<int64_t>(__shfl_xor(tmax, off, 64)));
    }
    if (lane == 0) {
      red_min[wave] = tmin;
      red_max[wave] = tmax;
    }
    // time tables in the base-2 domain
    for (int i = tid; i < 64; i += NT) {
      tb_lin[i] = -kLog2e * a.time_bias[min(i, a.nb - 1)];
      if (i < 32) tb_clz[i] = -kLog2e * a.time_bias[min(31 - i, a.nb - 1)];  // clz i <=> bucket 31-i
    }
    __syncthreads();
    tmin = red_min[0];
    tmax = red_max[0];
#pragma unroll
    for (int w = 1; w < HPB; ++w) {
      tmin = min(tmin, red_min[w]);
      tmax = max(tmax, red_max[w]);
    }
    c.tb_lo = static_cast<uint32_t>(tmin);
    // |dt| + 1 must fit 31 bits for the 32-bit path
    c.wide = (static_cast<uint64_t>(tmax) - static_cast<uint64_t>(tmin)) >= (1ull << 31) - 1;
  }

  const int n_kt = (c.nkeys + kBN - 1) / kBN;
  // key tiles made only of targets that are not queries of this block are
  // invisible to the whole block: a contiguous run [skip_a, skip_b)
  const int skip_a = (c.nc + c.first_tgt + kBN - 1) / kBN;
  const int skip_b = max((c.nc + q0) / kBN, skip_a);
  const int n_skip = skip_b - skip_a;
  const int n_steps = n_kt - n_skip;
  auto tile_of = [=](int st) { return st < skip_a ? st : st + n_skip; };
  // key steps [st_lo, st_hi) of this unit's chunk
  int st_lo, st_hi;
  chunk_range(n_steps, a.splits, chunk, st_lo, st_hi);
  // partial outputs of split items go to their chunk's slice of a.partial
  float* __restrict__ out = a.splits > 1 ? a.partial + static_cast<int64_t>(chunk) * a.total_tokens * a.d_model
                                         : a.av;

  // ---- per-slot query data of the bias builder ----
  SlotQ<SPT> sq;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int slot = tid + i * NT;
    const int qi = q0 + (slot >> 8) * 32 + (slot & 31);
    sq.qi[i] = qi;
    sq.pq[i] = c.nc + min(qi, c.first_tgt);
    const int64_t tq = a.ts[si.s + min(qi, si.L - 1)];
    sq.tq[i] = tq;
    sq.uq[i] = static_cast<uint32_t>(tq) - c.tb_lo;
  }

  // ---- Q fragments (B operand of S^T = K Q^T), prescaled by -alpha*log2(e) ----
  // lane: query qb*32 + lane%32, dims 16c + 8(lane/32) .. +7 of this head
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const float qscale = -a.alpha * kLog2e;
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = q0 + qb * 32 + (lane & 31);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (qi < si.L)
        raw = *reinterpret_cast<const uint4*>(Q + (si.s + qi) * c.d + c.col0 + hcol + cc * 16 +
                                              8 * (lane >> 5));
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(bf2f(w[e] & 0xffff) * qscale, bf2f(w[e] >> 16) * qscale);
      qf[qb][cc] = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // wave-uniform DMA row bases of this head group: block key kk is row
  // base + kk*d (own rows shifted back by the cache length)
  const uint16_t* kbase_o = static_cast<const uint16_t*>(a.k) + (c.s - c.nc) * c.d + c.col0;
  const uint16_t* vbase_o = static_cast<const uint16_t*>(a.v) + (c.s - c.nc) * c.d + c.col0;
  const uint16_t* kbase_c = a.ck ? static_cast<const uint16_t*>(a.ck) + c.cs * c.d + c.col0 : kbase_o;
  const uint16_t* vbase_c = a.cv ? static_cast<const uint16_t*>(a.cv) + c.cs * c.d + c.col0 : vbase_o;

  // per-lane LDS offsets of the MFMA operands
  const int g16 = lane >> 4;            // 16-lane group of the transposing reads
  const int sl = lane & 15;
  const int h2 = lane >> 5;             // half of the wave
  // A operand K: row lane%32, dims 16c + 8*h2 of this head
  const int koff = (lane & 31) * ROWBK + (hcol + 8 * h2) * 2;
  // B operand V (transposing read): source lane sl reads row 4*h2 + sl/4
  // (+8, +16*kh), dims 32db + 16*(g16&1) + 4*(sl&3)
  const int voff = (4 * h2 + (sl >> 2)) * ROWBV + (hcol + 16 * (g16 & 1) + 4 * (sl & 3)) * 2;

  if (st_lo < st_hi) {
  constexpr int RPW = kBN / HPB;   // DMA rows per wave of a K or V tile
#define SK(i) ((i) ? sK1 : sK0)
#define SV(i) ((i) ? sV1 : sV0)
#define SB(i) ((i) ? sB1 : sB0)
#define SD(i) ((i) ? &sD1 : &sD0)
  // ---- prologue: key data of tiles lo and lo+1, K/V rows and bias of tile lo ----
  load_keydata<HPB>(c, a.ts, a.c_ts, a.pos_bias, sD0, tile_of(st_lo), wave, lane);
  load_keydata<HPB>(c, a.ts, a.c_ts, a.pos_bias, sD1, tile_of(min(st_lo + 1, st_hi - 1)), wave, lane);
  {
    const int k0 = tile_of(st_lo) * kBN;
#pragma unroll
    for (int it = 0; it < RPW; ++it) {
      dma_row<HPB, ROWBK>(c, kbase_o, kbase_c, sK0, k0, wave + it * HPB, lane);
      dma_row<HPB, ROWBV>(c, vbase_o, vbase_c, sV0, k0, wave + it * HPB, lane);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  build_bias<HPB>(c, sq, sD0, sB0, tb_clz, tb_lin, a.nb, tile_of(st_lo), tid);
  __syncthreads();

  // Software pipeline in half tiles. Registers carried from step st-1 to
  // step st: the scores of the second 32-query block of tile st-1 (s1) and
  // the V operand of tile st-1 (vf). Step st (attn_step), buffers (st-lo)&1:
  //  A0. LDS reads for the bias of tile st+1 (first, so that their dependent
  //      time-bias lookups are not queued behind the big reads); DMA of the
  //      key data of tile st+2 and of the K/V rows of tile st+1 (over A0 and
  //      the first half of R0);
  //  R0. SiLU of s1 in quarters and O1 += P V_{st-1}; each consumed quarter of
  //      s1 is refilled with the block-1 bias of tile st and each consumed
  //      half of vf with V of tile st; the score MFMAs of block 0 of tile st
  //      into s0 (K and its bias read in the first quarter) in the second
  //      half; the bias of tile st+1 is finished and stored;
  //  R1. SiLU of s0 and O0 += P V_st, overlapped with the score MFMAs of
  //      block 1 into s1.
  // After the last step, a drain runs the SiLU and P.V of s1.
  // s1 and vf start at zero: the first step's R0 then adds exactly zero.
  f32x16 s0, s1;
  bf16x8 vf[2][2];
#pragma unroll
  for (int r = 0; r < 16; ++r) s1[r] = 0.f;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) vf[db][kh] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  // steps alternate between the two buffer sets
#define HSTU_ATTN_STEP(MORE, K0, B0, V0, K1, V1, B1, D1, D0)                                          \
  attn_step<HPB, MORE>(c, sq, a, st, st_hi, skip_a, n_skip, K0, B0, V0, K1, V1, B1, D1, D0, tb_clz,  \
                       tb_lin, kbase_o, kbase_c, vbase_o, vbase_c, qf, acc, s0, s1, vf, koff, voff,      \
                       wave, lane, tid)
  int st = st_lo;
#pragma clang loop unroll(disable)
  for (; st + 1 < st_hi; ++st) {
    const int p = (st - st_lo) & 1;
    HSTU_ATTN_STEP(true, SK(p), SB(p), SV(p), SK(p ^ 1), SV(p ^ 1), SB(p ^ 1), SD(p ^ 1), SD(p));
  }
  {
    const int p = (st - st_lo) & 1;
    HSTU_ATTN_STEP(false, SK(p), SB(p), SV(p), SK(p ^ 1), SV(p ^ 1), SB(p ^ 1), SD(p ^ 1), SD(p));
  }
  // drain: SiLU and P.V of block 1 of the last tile
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const bf16x8 pk = silu8(s1, kh);
#pragma unroll
    for (int db = 0; db < 2; ++db) acc[1][db] = mfma32(pk, vf[db][kh], acc[1][db]);
  }
  }   // non-empty chunk
#undef SK
#undef SV
#undef SB
#undef SD
#undef HSTU_ATTN_STEP

  if constexpr (FUSE_NG) {
    // ---- fused norm_gate: the 64 x d AV tile (AV = -ln2 * O) goes to LDS,
    // then each wave turns whole rows into G with the norm_gate row code.
    // U of a batch of up to 8 rows per wave is loaded ahead of the LDS pass,
    // so its latency overlaps the tile transfer ----
    constexpr int TD = HPB * kDH;   // = d_model: one head group covers the row
    constexpr int RPW = kBM / HPB;  // rows per wave
    constexpr int RB = RPW < 8 ? RPW : 8;
    const uint16_t* __restrict__ ng_u = static_cast<const uint16_t*>(a.ng_u);
    __syncthreads();   // every wave is done with the K/V buffers
    uint2 ur[RB][kNgMaxChunks];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int qi = min(q0 + wave + b * HPB, si.L - 1);
      load_u_chunks_bf16(ng_u + (si.s + qi) * TD, TD, lane, ur[b]);
    }
    float* tile = reinterpret_cast<float*>(skv);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
#pragma unroll
        for (int db = 0; db < 2; ++db) tile[row * TD + hcol + db * 32 + (lane & 31)] = -kLn2 * acc[qb][db][r];
      }
    __syncthreads();
    for (int b0 = 0; b0 < RPW; b0 += RB) {
      if (b0 > 0) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int qi = min(q0 + wave + (b0 + b) * HPB, si.L - 1);
          load_u_chunks_bf16(ng_u + (si.s + qi) * TD, TD, lane, ur[b]);
        }
      }
      const float* avr[RB];
      uint16_t* g[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int rr = wave + (b0 + b) * HPB;
        avr[b] = tile + rr * TD;
        g[b] = q0 + rr < si.L ? static_cast<uint16_t*>(a.ng_g) + (si.s + q0 + rr) * TD : nullptr;
      }
      norm_gate_rows_bf16<RB>(avr, ur, g, TD, a.ng_eps, a.ng_gamma, a.ng_beta, lane);
    }
  } else {
  // ---- AV = -ln2 * O: lane -> query qb*32 + 8(r/4) + 4*h2 + r%4, dim 32db + lane%32 ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = q0 + qb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
      if (qi < si.L) {
        float* row = out + (si.s + qi) * c.d + c.col0 + hcol + (lane & 31);
#pragma unroll
        for (int db = 0; db < 2; ++db) row[db * 32] = -kLn2 * acc[qb][db][r];
      }
    }
  }
  }   // work items
}

// fp32 kernel: one thread per query row, plain FMA loops, exact expf and IEEE
// division. It serves the fp32 dtype (small workloads). Keys arrive in
// chunks of 64 staged in LDS by the whole workgroup, so a thread's loop over
// keys does not wait on global memory at every key.
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float sk[64][DH];
  __shared__ float sv[64][DH];
  __shared__ int64_t skt[64];
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
  for (int k0 = 0; k0 < nkeys; k0 += 64) {
    __syncthreads();   // the previous chunk's reads are done
    for (int i = threadIdx.x; i < 64 * DH; i += 64) {
      const int r = i / DH, cc = i - r * DH;
      const int kk = k0 + r;
      float kv = 0.0f, vv = 0.0f;
      if (kk < nkeys) {
        const bool cache = kk < si.nc;
        const int64_t row = cache ? (si.cs + kk) : (si.s + kk - si.nc);
        kv = (cache ? CK : K)[row * d + h * DH + cc];
        vv = (cache ? CV : V)[row * d + h * DH + cc];
      }
      sk[r][cc] = kv;
      sv[r][cc] = vv;
    }
    {
      const int kk = k0 + threadIdx.x;
      skt[threadIdx.x] = kk < nkeys ? (kk < si.nc ? a.c_ts[si.cs + kk] : a.ts[si.s + kk - si.nc]) : 0;
    }
    __syncthreads();
    const int kend = min(64, nkeys - k0);
    for (int r = 0; r < kend; ++r) {
      const int kk = k0 + r;
      const bool cache = kk < si.nc;
      const int j = kk - si.nc;
      const bool vis = qvalid && (cache || ((j <= qi) && (j < first_tgt ||
                                                        (j == qi && !(a.no_self && qi >= first_tgt)))));
      if (!vis) continue;
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < DH; ++c) dot = fmaf(qv[c], sk[r][c], dot);
      const int pk = cache ? kk : si.nc + (j < first_tgt ? j : first_tgt);
      int pidx = pq - pk + a.pos_center;
      pidx = pidx < 0 ? 0 : (pidx >= a.pos_len ? a.pos_len - 1 : pidx);
      const float s = a.alpha * dot + a.pos_bias[pidx] + a.time_bias[time_bucket64(tq - skt[r], a.nb)];
      const float w = s / (1.0f + expf(-s));
#pragma unroll
      for (int c = 0; c < DH; ++c) acc[c] = fmaf(w, sv[r][c], acc[c]);
    }
  }
  if (qvalid) {
#pragma unroll
    for (int c = 0; c < DH; ++c) a.av[(si.s + qi) * d + h * DH + c] = acc[c];
  }
}

}  // namespace

bool attn_can_fuse_norm_gate(int num_heads, int num_seqs, int max_seq_len) {
  // one head group (8, 4, 2 or 1 heads) per row, and no key-range splits
  return (num_heads == 8 || num_heads == 4 || num_heads == 2 || num_heads == 1) &&
         attn_splits(num_seqs, max_seq_len) == 1;
}

int attn_splits(int num_seqs, int max_seq_len) {
  const int64_t items = static_cast<int64_t>(num_seqs) * ((static_cast<int64_t>(max_seq_len) + kBM - 1) / kBM);
  if (items <= 0 || items >= kSplitMinUnits) return 1;
  return static_cast<int>(std::min<int64_t>(kMaxSplits, (kSplitMinUnits + items - 1) / items));
}

size_t attn_sched_bytes(int num_seqs, int max_seq_len) {
  const int64_t n_qt = (static_cast<int64_t>(max_seq_len) + kBM - 1) / kBM;
  const int64_t units = static_cast<int64_t>(num_seqs) * n_qt * attn_splits(num_seqs, max_seq_len);
  const size_t bytes = static_cast<size_t>(kSchedHead + units) * sizeof(int);
  return (bytes + 255) & ~static_cast<size_t>(255);
}

size_t attn_workspace_bytes(int num_seqs, int max_seq_len, int64_t total_tokens, int d_model) {
  const int S = attn_splits(num_seqs, max_seq_len);
  const size_t partial = S > 1 ? static_cast<size_t>(S) * total_tokens * d_model * sizeof(float) : 0;
  return attn_sched_bytes(num_seqs, max_seq_len) + partial;
}

// AV = sum over chunks of the partial outputs, in chunk order (deterministic).
__global__ __launch_bounds__(256) void attn_reduce_kernel(const float* __restrict__ partial,
                                                          float* __restrict__ av, int64_t n4,
                                                          int64_t stride4, int splits) {
  const float4* p = reinterpret_cast<const float4*>(partial);
  float4* o = reinterpret_cast<float4*>(av);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float4 acc = p[i];
    for (int c = 1; c < splits; ++c) {
      const float4 v = p[c * stride4 + i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    o[i] = acc;
  }
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.max_seq_len + kBM - 1) / kBM;
  if (a.num_seqs == 0 || n_qt == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(1024), 0, s, a, n_qt);
  int hpb = 1;
  for (int c : {8, 4, 2, 1})
    if (a.num_heads % c == 0) {
      hpb = c;
      break;
    }
  // a multiple of the XCD count, one workgroup per unit on average
  const int64_t units = static_cast<int64_t>(a.num_seqs) * n_qt * a.splits;
  dim3 grid(static_cast<unsigned>((units + kNumXcd - 1) / kNumXcd * kNumXcd), a.num_heads / hpb);
  if (a.fuse_ng) {
    if (!attn_can_fuse_norm_gate(a.num_heads, a.num_seqs, a.max_seq_len) || a.splits != 1)
      return hipErrorInvalidValue;
    switch (hpb) {
      case 8: hipLaunchKernelGGL((attn_bf16_kernel<8, true>), grid, dim3(512), 0, s, a); break;
      case 4: hipLaunchKernelGGL((attn_bf16_kernel<4, true>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((attn_bf16_kernel<2, true>), grid, dim3(128), 0, s, a); break;
      default: hipLaunchKernelGGL((attn_bf16_kernel<1, true>), grid, dim3(64), 0, s, a); break;
    }
    return hipGetLastError();
  }
  switch (hpb) {
    case 8: hipLaunchKernelGGL((attn_bf16_kernel<8, false>), grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_bf16_kernel<4, false>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_bf16_kernel<2, false>), grid, dim3(128), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_bf16_kernel<1, false>), grid, dim3(64), 0, s, a); break;
  }
  if (a.splits > 1) {
    const int64_t n4 = a.total_tokens * a.d_model / 4;
    const int blocks = static_cast<int>(std::min<int64_t>((n4 + 255) / 256, 4096));
    if (n4 > 0)
      hipLaunchKernelGGL(attn_reduce_kernel, dim3(blocks), dim3(256), 0, s, a.partial, a.av, n4, n4,
                         a.splits);
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
