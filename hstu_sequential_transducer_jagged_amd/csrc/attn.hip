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
//    (global_load_lds_dwordx4, written as inline assembly so that the
//    compiler's waits for LDS reads ignore them) into a double buffer: the
//    step's barrier sits between its two halves, and the loads of tile st+2
//    go into tile st's buffers right after it, with a whole step to land;
//  * the relative bias is shared by all heads: the workgroup builds each
//    64 x 32 bias tile once, two steps ahead, from per-key timestamps staged in
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
//    cores and the vector ALUs of a wave overlap; the loads of a tile are
//    spread over the second half of the step;
//  * time buckets are exact integers: 32-bit |dt|+1 and a leading-zero count
//    when every pair of the tile is within 2^30 s of the block's reference
//    time, a 64-bit path otherwise.
#include "common.h"
#include "internal.h"
#include "attn_sched.h"

#include <algorithm>
#include <mutex>

namespace hstu {
namespace {

constexpr int kBM = kAttnBM;   // query rows per workgroup
constexpr int kBN = kAttnBN;   // keys per step
using sched::chunk_range;
using sched::kListInts;
using sched::kNumXcd;
using sched::kSchedHead;
using sched::seq_info;
using sched::SeqInfo;
using sched::tile_steps;
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

// Direct global->LDS loads written as inline assembly. The compiler does
// not see their LDS writes, so it neither holds LDS reads of other buffers
// behind them nor turns its waits for ordinary LDS reads into full drains.
// The kernel orders every reader after them itself: an explicit
// s_waitcnt vmcnt(0), then a workgroup barrier. M0 carries the wave's LDS
// destination (one wait state between its write and the load); the loads
// have no register results.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(const void, p)));
}
// 16 bytes per lane from row + voff into LDS [lds + 16 lane, +16)
__device__ __forceinline__ void dma_b128(const void* row, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(row)
               : "memory", "m0");
}
// 4 bytes per lane from src into LDS [lds + 4 lane, +4)
__device__ __forceinline__ void dma_b32(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}

// Bias modes of the bf16 kernel (template parameter): the position and time
// tables; the tables with one time table per (query type, key type) pair;
// the parameter-free bias -m_p dp - m_t bucket computed from the two slopes.
constexpr int kBiasTables = 0;
constexpr int kBiasTyped = 1;
constexpr int kBiasLinear = 2;
constexpr int kMaxTypePairs = 16;    // up to 4 token types

// Per-key data of one key tile, delivered to LDS by DMA two tiles ahead.
struct KeyData {
  alignas(16) uint32_t tlo[kBN];    // low words of the key timestamps
  alignas(16) uint32_t thi[kBN];    // high words (64-bit path)
  alignas(16) float pos[kPosWin];   // raw position-bias window, entry e <-> dp = w0 + e
  alignas(16) int32_t ty[kBN];      // key token types (typed mode)
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

// DMA of a tile's key data, four items: 0 the timestamps (lanes 0..31 low
// words, 32..63 high words), 1 and 2 the halves of the position window
// (table modes), 3 the key types (typed mode); item i is issued by wave
// i % HPB. Key types outside [0, nt) are clamped where they are used.
template <int HPB, int MODE>
__device__ __forceinline__ void load_keydata(const Ctx& c, const AttnArgs& a, KeyData& kd, int tile, int wave,
                                             int lane) {
#pragma unroll
  for (int item = 0; item < 4; ++item) {
    if (item % HPB != wave) continue;
    if (item == 0) {
      const int kk = min(tile * kBN + (lane & (kBN - 1)), c.nkeys - 1);
      const int64_t* tp = kk < c.nc ? a.c_ts + (c.cs + kk) : a.ts + (c.s + kk - c.nc);
      const uint32_t* src = reinterpret_cast<const uint32_t*>(tp) + (lane >> 5);
      dma_b32(src, lds_addr(kd.tlo));
    } else if (item <= 2) {
      if (MODE == kBiasLinear) continue;
      const int half = item - 1;
      int idx = c.pos_center + window_origin(c, tile) + half * 64 + lane;
      idx = idx < 0 ? 0 : (idx >= c.pos_len ? c.pos_len - 1 : idx);
      dma_b32(a.pos_bias + idx, lds_addr(kd.pos + half * 64));
    } else {
      if (MODE != kBiasTyped) continue;
      if (lane < kBN) {
        const int kk = min(tile * kBN + lane, c.nkeys - 1);
        const int32_t* src = kk < c.nc ? a.c_types + (c.cs + kk) : a.types + (c.s + kk - c.nc);
        dma_b32(src, lds_addr(kd.ty));
      }
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
  dma_b128(src, static_cast<uint32_t>(lane) * 16u, lds_addr(dst + r * ROWB));
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
  int ty[SPT];          // query token type x nt (typed mode)
};

// Base-2 bias of one pair from its time bucket (as the clz of |dt|+1 on the
// 32-bit path, or the bucket itself on the 64-bit one) and, per mode, the
// position-table value or the position difference:
//   tables: -log2(e) (pb + tb[type pair][bucket]);
//   linear: log2(e) (m_p dp + m_t bucket).
// tb_clz / tb_lin hold -log2(e) times the time tables, indexed by
// (type pair) * 32 + clz and (type pair) * 64 + bucket.
template <int MODE>
__device__ __forceinline__ float pair_bias_clz(const AttnArgs& a, const float* tb_clz, int tp, uint32_t clz,
                                               float pb_or_dp) {
  if constexpr (MODE == kBiasLinear) {
    const int bucket = min(31 - static_cast<int>(clz), a.nb - 1);
    return kLog2e * __builtin_fmaf(a.m_p, pb_or_dp, a.m_t * static_cast<float>(bucket));
  } else {
    return __builtin_fmaf(pb_or_dp, -kLog2e, tb_clz[tp * 32 + clz]);
  }
}

// Bias tile (base-2 domain) of key tile `tile` from its key data.
template <int HPB, int MODE>
__device__ __forceinline__ void build_bias(const Ctx& c, const AttnArgs& a, const SlotQ<512 / (64 * HPB)>& sq,
                                           const KeyData& kd, float* bias, const float* tb_clz,
                                           const float* tb_lin, int tile, int tid) {
  constexpr int NT = 64 * HPB;
  constexpr int SPT = 512 / NT;
  const int k0 = tile * kBN;
  const int w0 = window_origin(c, tile);
  const int nb = a.nb, nt = a.ntypes;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int slot = tid + i * NT;
    const int kr = 8 * ((slot >> 6) & 3) + 4 * ((slot >> 5) & 1);
    const int kbase = k0 + kr;
    const int qi = sq.qi[i];
    float b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = kbase + r;
      const int jo = kk - c.nc;
      const bool vis = qi < c.L && kk < c.nkeys &&
                       (kk < c.nc ||
                        (jo <= qi && (jo < c.first_tgt || (jo == qi && !(c.no_self && qi >= c.first_tgt)))));
      const int dp = sq.pq[i] - key_pos(kk, c.nc, c.first_tgt);
      int tp = 0;
      if constexpr (MODE == kBiasTyped) tp = sq.ty[i] + min(max(kd.ty[kr + r], 0), nt - 1);
      float pv;
      if constexpr (MODE == kBiasLinear) {
        pv = static_cast<float>(dp);
      } else {
        int pidx = dp - w0;
        pidx = pidx < 0 ? 0 : (pidx >= kPosWin ? kPosWin - 1 : pidx);
        pv = kd.pos[pidx];
      }
      float bv;
      if (!c.wide) {
        const uint32_t x = sq.uq[i], y = kd.tlo[kr + r] - c.tb_lo;
        const uint32_t ad = (x > y ? x - y : y - x) + 1u;
        bv = pair_bias_clz<MODE>(a, tb_clz, tp, __builtin_clz(ad), pv);
      } else {
        const int64_t tk = static_cast<int64_t>((static_cast<uint64_t>(kd.thi[kr + r]) << 32) | kd.tlo[kr + r]);
        const int bucket = time_bucket64(sq.tq[i] - tk, nb);
        if constexpr (MODE == kBiasLinear)
          bv = kLog2e * __builtin_fmaf(a.m_p, pv, a.m_t * static_cast<float>(bucket));
        else
          bv = __builtin_fmaf(pv, -kLog2e, tb_lin[tp * 64 + bucket]);
      }
      b[r] = vis ? bv : kMaskBias;
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
  float pw[SPT][4];     // position-table values (table modes) or position differences (linear)
  float tb[SPT][4];
  int ty[SPT][4];       // key types (typed mode)
};

template <int HPB, int MODE>
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
    if constexpr (MODE == kBiasTyped) {
      const int4 y4 = *reinterpret_cast<const int4*>(&kd.ty[kr]);
      fb.ty[i][0] = y4.x;
      fb.ty[i][1] = y4.y;
      fb.ty[i][2] = y4.z;
      fb.ty[i][3] = y4.w;
    }
    if constexpr (MODE == kBiasLinear) {
#pragma unroll
      for (int r = 0; r < 4; ++r) fb.pw[i][r] = static_cast<float>(sq.pq[i] - (k0 + kr + r));   // p_k = kk
    } else {
      int pb = sq.pq[i] - (k0 + kr) - w0;   // p_k = kk for non-target keys
      pb = pb < 3 ? 3 : (pb > kPosWin - 1 ? kPosWin - 1 : pb);
#pragma unroll
      for (int r = 0; r < 4; ++r) fb.pw[i][r] = kd.pos[pb - r];
    }
  }
}

template <int HPB, int MODE>
__device__ __forceinline__ void fast_bias_lookup(const Ctx& c, const AttnArgs& a, const SlotQ<512 / (64 * HPB)>& sq,
                                                 const float* tb_clz, FastBias<512 / (64 * HPB)>& fb) {
  constexpr int SPT = 512 / (64 * HPB);
#pragma unroll
  for (int i = 0; i < SPT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t x = sq.uq[i], y = fb.tk[i][r] - c.tb_lo;
      const uint32_t ad = (x > y ? x - y : y - x) + 1u;   // |dt| + 1 >= 1
      const uint32_t clz = __builtin_clz(ad);
      if constexpr (MODE == kBiasLinear) {
        fb.tb[i][r] = a.m_t * static_cast<float>(min(31 - static_cast<int>(clz), a.nb - 1));
      } else {
        int tp = 0;
        if constexpr (MODE == kBiasTyped) tp = sq.ty[i] + min(max(fb.ty[i][r], 0), a.ntypes - 1);
        fb.tb[i][r] = tb_clz[tp * 32 + clz];
      }
    }
}

template <int HPB, int MODE>
__device__ __forceinline__ void fast_bias_store(const AttnArgs& a, const FastBias<512 / (64 * HPB)>& fb, float* bias,
                                                int tid) {
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
      if constexpr (MODE == kBiasLinear)
        b[r] = kLog2e * __builtin_fmaf(a.m_p, fb.pw[i][r], tb);
      else
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

// One key step of the software pipeline (see the kernel). The step reads
// the K, V and bias tiles of tile st (cur*) before its barrier; after it,
// every wave has read them, so the same buffers take the K/V rows and the
// bias of tile st+2, and keyD (key data of tile st+3) replaces the key data
// of tile st+1. The loads of tile st+2 then have until the barrier of step
// st+1, a whole step, to land. AHEAD: 2 when tile st+2 exists (barrier,
// loads and bias), 1 for the step before the last (barrier only: tile st+1
// is landing), 0 for the last step. Key data past the chunk's last tile is
// clamped to it (a few bytes, into a buffer that is not read again). FIRST:
// the chunk's first step, which also builds the bias of tile st+1 into the
// other buffer (othB, from the key data in othD) before its barrier.
template <int HPB, int AHEAD, bool FIRST, int MODE>
__device__ __forceinline__ void attn_step(
    const Ctx& c, const SlotQ<512 / (64 * HPB)>& sq, const AttnArgs& a, int st, int st_hi, int skip_a,
    int n_skip, uint8_t* __restrict__ curK, float* __restrict__ curB, uint8_t* __restrict__ curV,
    const KeyData* __restrict__ biasD, KeyData* __restrict__ keyD, float* __restrict__ othB,
    const KeyData* __restrict__ othD, const float* __restrict__ tb_clz,
    const float* __restrict__ tb_lin, const uint16_t* kbase_o, const uint16_t* kbase_c, const uint16_t* vbase_o,
    const uint16_t* vbase_c, const bf16x8 (&qf)[2][4], f32x16 (&acc)[2][2], f32x16& s0, f32x16& s1,
    bf16x8 (&vf)[2][2], int koff, int voff, int wave, int lane, int tid) {
  constexpr int ROWBV = Rows<HPB>::ROWBV;
  // R0: SiLU of block 1 of tile st-1 in quarters, each quarter's registers
  // then refilled with the block-1 bias of tile st; P.V with V of tile
  // st-1, each half of vf then refilled with V of tile st; the score MFMAs
  // of block 0 in the second half
  bf16x8 kf[4];
  {
    uint32_t w[8];
    silu4(s1, 0, w[0], w[1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      kf[cc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(curK + koff + cc * 32));
    load_bias_block(curB, 0, lane, s0);
    load_bias_quarter(curB, 1, 0, lane, s1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sr = 1; sr < 4; ++sr) {
      silu4(s1, sr, w[2 * sr], w[2 * sr + 1]);
      load_bias_quarter(curB, 1, sr, lane, s1);
      if (sr >= 2) {
        s0 = mfma32(kf[2 * (sr - 2)], qf[0][2 * (sr - 2)], s0);
        s0 = mfma32(kf[2 * (sr - 2) + 1], qf[0][2 * (sr - 2) + 1], s0);
      }
      if (sr & 1) {
        const int kh = sr >> 1;
        const bf16x8 pk = __builtin_bit_cast(bf16x8, make_uint4(w[4 * kh], w[4 * kh + 1], w[4 * kh + 2], w[4 * kh + 3]));
#pragma unroll
        for (int db = 0; db < 2; ++db) acc[1][db] = mfma32(pk, vf[db][kh], acc[1][db]);
        load_v_half<ROWBV>(curV, voff, kh, vf);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(w[7]));
  }
  if (FIRST && AHEAD >= 1) {
    const int s1t = st + 1 < skip_a ? st + 1 : st + 1 + n_skip;
    build_bias<HPB, MODE>(c, a, sq, *othD, othB, tb_clz, tb_lin, s1t, tid);
  }
  // the barrier: every wave has read tile st's buffers, and the loads of
  // tile st+1 and of the key data of tile st+2 (issued one step earlier)
  // have landed
  constexpr bool MORE = AHEAD == 2;
  int t2 = 0;
  bool fast2 = false;
  FastBias<512 / (64 * HPB)> fb;
  if (AHEAD >= 1) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (MORE) {
    const int s2 = st + 2;
    t2 = s2 < skip_a ? s2 : s2 + n_skip;
    // the bias of tile t2 takes the split fast path when all its keys are
    // visible non-targets for the whole block and times fit 32 bits
    const int k2 = t2 * kBN;
    fast2 = (k2 + kBN - 1 - c.nc <= c.q0) && (k2 + kBN - 1 - c.nc < c.first_tgt) && !c.wide;
    fast_bias_issue<HPB, MODE>(c, sq, *biasD, t2, tid, fb);
    const int s3 = min(st + 3, st_hi - 1);
    load_keydata<HPB, MODE>(c, a, *keyD, s3 < skip_a ? s3 : s3 + n_skip, wave, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  // R1: SiLU of block 0 of tile st and its P.V; the score MFMAs of block 1;
  // the K/V rows of tile t2, two loads per quarter (issued faster, they
  // stall the wave; issued later, they land late); the time-bias lookups
  // of tile t2 after the first quarter and their combine and store after the
  // last
  {
    uint32_t w[8];
#pragma unroll
    for (int sr = 0; sr < 4; ++sr) {
      silu4(s0, sr, w[2 * sr], w[2 * sr + 1]);
      if (MORE && sr == 1) fast_bias_lookup<HPB, MODE>(c, a, sq, tb_clz, fb);
      if (MORE) {
        dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, curK, curV, t2 * kBN, 2 * sr, wave, lane);
        dma_slot<HPB>(c, kbase_o, kbase_c, vbase_o, vbase_c, curK, curV, t2 * kBN, 2 * sr + 1, wave, lane);
      }
      if (MORE && sr == 3) fast_bias_store<HPB, MODE>(a, fb, curB, tid);
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
    asm volatile("" ::"v"(w[7]));
  }
  // tiles off the fast path: the full bias builder overwrites the tile
  if (MORE && !fast2) build_bias<HPB, MODE>(c, a, sq, *biasD, curB, tb_clz, tb_lin, t2, tid);
}

// The scheduling pass in its own launch: one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void attn_schedule_kernel(AttnArgs a, int n_qt) {
  __shared__ int cnt[kListInts];
  __shared__ long long wsum[16];
  sched::build<1024>(a, n_qt, cnt, wsum);
}

template <int HPB, bool FUSE_NG, int MODE>
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
  // base-2 time tables: (type pair) * 32 + clz(|dt|+1) and (type pair) * 64 + bucket
  constexpr int kPairs = MODE == kBiasTyped ? kMaxTypePairs : 1;
  __shared__ float tb_clz[kPairs * 32];
  __shared__ float tb_lin[kPairs * 64];
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
  const int n_qt = (a.max_seq_len + a.bm - 1) / a.bm;
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
    if (MODE != kBiasLinear) {
      const int pairs = MODE == kBiasTyped ? a.ntypes * a.ntypes : 1;
      for (int i = tid; i < pairs * 64; i += NT) {
        const int tp = i >> 6, b = i & 63;
        tb_lin[i] = -kLog2e * a.time_bias[tp * a.nb + min(b, a.nb - 1)];
        if (b < 32)   // clz b <=> bucket 31 - b
          tb_clz[tp * 32 + b] = -kLog2e * a.time_bias[tp * a.nb + min(31 - b, a.nb - 1)];
      }
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
    sq.ty[i] = MODE == kBiasTyped ? min(max(a.types[si.s + min(qi, si.L - 1)], 0), a.ntypes - 1) * a.ntypes : 0;
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
  // ---- prologue: key data and K/V rows of tiles lo and lo+1 (key data of
  // tile t in buffer (t - lo) & 1), the bias of tile lo, then the key data
  // of tile lo+2 ----
  const bool two = st_lo + 1 < st_hi;
  load_keydata<HPB, MODE>(c, a, sD0, tile_of(st_lo), wave, lane);
  if (two) load_keydata<HPB, MODE>(c, a, sD1, tile_of(st_lo + 1), wave, lane);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1 && !two) break;
    const int k0 = tile_of(st_lo + t) * kBN;
#pragma unroll
    for (int it = 0; it < RPW; ++it) {
      dma_row<HPB, ROWBK>(c, kbase_o, kbase_c, SK(t), k0, wave + it * HPB, lane);
      dma_row<HPB, ROWBV>(c, vbase_o, vbase_c, SV(t), k0, wave + it * HPB, lane);
    }
  }
  // the K/V rows of tile lo+1 (this wave's last 2 RPW loads) may still be
  // landing while bias lo is built; the first step's barrier waits for them
  if (two) {
    constexpr int kLate = 2 * RPW < 63 ? 2 * RPW : 63;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLate) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  build_bias<HPB, MODE>(c, a, sq, sD0, sB0, tb_clz, tb_lin, tile_of(st_lo), tid);
  __syncthreads();
  if (st_lo + 2 < st_hi) load_keydata<HPB, MODE>(c, a, sD0, tile_of(st_lo + 2), wave, lane);

  // Software pipeline in half tiles. Registers carried from step st-1 to
  // step st: the scores of the second 32-query block of tile st-1 (s1) and
  // the V operand of tile st-1 (vf). Step st (attn_step) uses buffer set
  // p = (st-lo)&1 for the K, V and bias tiles of tile st:
  //  R0. SiLU of s1 in quarters and O1 += P V_{st-1}; each consumed quarter of
  //      s1 is refilled with the block-1 bias of tile st and each consumed
  //      half of vf with V of tile st; the score MFMAs of block 0 of tile st
  //      into s0 (K and its bias read in the first quarter) in the second
  //      half;
  //  barrier: set p is free, tile st+1 and the key data of tile st+2 have
  //      landed;
  //  R1. SiLU of s0 and O0 += P V_st, overlapped with the score MFMAs of
  //      block 1 into s1; the K/V rows of tile st+2 go into set p and its
  //      bias is built there (key data from buffer p), the key data of tile
  //      st+3 goes into buffer p^1.
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
#define HSTU_ATTN_STEP(AHEAD, FIRST, K, B, V, DB, DK)                                                     \
  attn_step<HPB, AHEAD, FIRST, MODE>(c, sq, a, st, st_hi, skip_a, n_skip, K, B, V, DB, DK, sB1, &sD1, tb_clz,  \
                                     tb_lin, kbase_o, kbase_c, vbase_o, vbase_c, qf, acc, s0, s1, vf, koff,   \
                                     voff, wave, lane, tid)
  int st = st_lo;
  // the first step also builds the bias of tile lo+1 before its barrier
  if (st + 2 < st_hi) {
    HSTU_ATTN_STEP(2, true, sK0, sB0, sV0, &sD0, &sD1);
    ++st;
  } else if (st + 1 < st_hi) {
    HSTU_ATTN_STEP(1, true, sK0, sB0, sV0, &sD0, &sD1);
    ++st;
  }
#pragma clang loop unroll(disable)
  for (; st + 2 < st_hi; ++st) {
    const int p = (st - st_lo) & 1;
    HSTU_ATTN_STEP(2, false, SK(p), SB(p), SV(p), SD(p), SD(p ^ 1));
  }
  if (st + 1 < st_hi) {
    const int p = (st - st_lo) & 1;
    HSTU_ATTN_STEP(1, false, SK(p), SB(p), SV(p), SD(p), SD(p ^ 1));
    ++st;
  }
  {
    const int p = (st - st_lo) & 1;
    HSTU_ATTN_STEP(0, false, SK(p), SB(p), SV(p), SD(p), SD(p ^ 1));
  }
  // the clamped key-data loads of the last full step may still be in flight
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

// Input element as fp32: fp32 as is, bf16 (raw 16-bit pattern) widened.
template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if constexpr (BF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  else
    return static_cast<const float*>(p)[i];
}

// fp32 kernel: one thread per query row, plain FMA loops, exact expf and IEEE
// division. It serves the fp32 dtype (small workloads) and, reading bf16
// inputs (BF16), the bf16 cases no matrix-core kernel takes: head_dim 32
// with targets, a cache, token types or the parameter-free bias. Keys arrive
// in chunks of 64 staged in LDS by the whole workgroup, so a thread's loop
// over keys does not wait on global memory at every key.
template <int DH, bool BF16>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float sk[64][DH];
  __shared__ float sv[64][DH];
  __shared__ int64_t skt[64];
  __shared__ int sty[64];
  const int seq = blockIdx.x;
  const int qt = blockIdx.y;
  const int h = blockIdx.z;
  const SeqInfo si = seq_info(a, seq);
  const int qi = qt * 64 + threadIdx.x;
  if (qt * 64 >= si.L) return;
  const bool qvalid = qi < si.L;
  const int d = a.d_model;
  const int first_tgt = si.L - si.m;
  float qv[DH], acc[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qv[c] = qvalid ? ld_in<BF16>(a.q, (si.s + qi) * d + h * DH + c) : 0.0f;
    acc[c] = 0.0f;
  }
  const int pq = si.nc + (qi < first_tgt ? qi : first_tgt);
  const int64_t tq = qvalid ? a.ts[si.s + qi] : 0;
  const int nt = a.ntypes;
  // token types outside [0, nt) are clamped (hstu_check_inputs reports them)
  const int tyq = nt > 1 && qvalid ? min(max(a.types[si.s + qi], 0), nt - 1) : 0;
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
        kv = ld_in<BF16>(cache ? a.ck : a.k, row * d + h * DH + cc);
        vv = ld_in<BF16>(cache ? a.cv : a.v, row * d + h * DH + cc);
      }
      sk[r][cc] = kv;
      sv[r][cc] = vv;
    }
    {
      const int kk = k0 + threadIdx.x;
      skt[threadIdx.x] = kk < nkeys ? (kk < si.nc ? a.c_ts[si.cs + kk] : a.ts[si.s + kk - si.nc]) : 0;
      sty[threadIdx.x] = nt > 1 && kk < nkeys
                             ? min(max(kk < si.nc ? a.c_types[si.cs + kk] : a.types[si.s + kk - si.nc], 0), nt - 1)
                             : 0;
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
      const int bucket = time_bucket64(tq - skt[r], a.nb);
      float rab;
      if (a.linear) {
        // the parameter-free bias -m_p (p_i - p_j) - m_t bucket
        rab = -a.m_p * static_cast<float>(pq - pk) - a.m_t * static_cast<float>(bucket);
      } else {
        int pidx = pq - pk + a.pos_center;
        pidx = pidx < 0 ? 0 : (pidx >= a.pos_len ? a.pos_len - 1 : pidx);
        rab = a.pos_bias[pidx] + a.time_bias[(tyq * nt + sty[r]) * a.nb + bucket];
      }
      const float s = a.alpha * dot + rab;
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

namespace {
template <bool FUSE_NG, int MODE>
void launch_attn_kernel(int hpb, dim3 grid, const AttnArgs& a, hipStream_t s) {
  switch (hpb) {
    case 8: hipLaunchKernelGGL((attn_bf16_kernel<8, FUSE_NG, MODE>), grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_bf16_kernel<4, FUSE_NG, MODE>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_bf16_kernel<2, FUSE_NG, MODE>), grid, dim3(128), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_bf16_kernel<1, FUSE_NG, MODE>), grid, dim3(64), 0, s, a); break;
  }
}
}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.max_seq_len + kBM - 1) / kBM;
  if (a.num_seqs == 0 || n_qt == 0) return hipSuccess;
  if (a.bm != kBM) return hipErrorInvalidValue;
  if (!a.sched_ready) hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(1024), 0, s, a, n_qt);
  // a multiple of the XCD count, one workgroup per unit on average
  const int64_t units = static_cast<int64_t>(a.num_seqs) * n_qt * a.splits;
  const unsigned gx = static_cast<unsigned>((units + kNumXcd - 1) / kNumXcd * kNumXcd);
  if (a.fuse_ng && (a.splits != 1 || !attn_can_fuse_norm_gate(a.num_seqs, a.max_seq_len, a.num_heads,
                                                              a.total_tokens, a.d_model)))
    return hipErrorInvalidValue;
  const int hpb = attn_heads_per_group(a.num_heads);
  const dim3 grid(gx, a.num_heads / hpb);
  const int mode = a.linear ? kBiasLinear : (a.ntypes > 1 ? kBiasTyped : kBiasTables);
  if (a.fuse_ng) {
    switch (mode) {
      case kBiasTyped: launch_attn_kernel<true, kBiasTyped>(hpb, grid, a, s); break;
      case kBiasLinear: launch_attn_kernel<true, kBiasLinear>(hpb, grid, a, s); break;
      default: launch_attn_kernel<true, kBiasTables>(hpb, grid, a, s); break;
    }
  } else {
    switch (mode) {
      case kBiasTyped: launch_attn_kernel<false, kBiasTyped>(hpb, grid, a, s); break;
      case kBiasLinear: launch_attn_kernel<false, kBiasLinear>(hpb, grid, a, s); break;
      default: launch_attn_kernel<false, kBiasTables>(hpb, grid, a, s); break;
    }
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

// Device scratch of the allocation-free attention entry point: the work
// list and the partial outputs of hstu_attn_fwd_noalloc. One copy per device
// (each device's code object holds its own), kept until the process ends.
// Host code never uses the array's name as an address: the device address
// comes from hipGetSymbolAddress, resolved once per device.
static __device__ __align__(256) unsigned char scratch[kAttnStaticScratchBytes];

hipError_t attn_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.max_seq_len + 63) / 64;
  if (a.num_seqs == 0 || n_qt == 0) return hipSuccess;
  dim3 grid(a.num_seqs, n_qt, a.num_heads);
  if (a.in_bf16 && a.head_dim != 32) return hipErrorInvalidValue;
  if (a.in_bf16)
    hipLaunchKernelGGL((attn_f32_kernel<32, true>), grid, dim3(64), 0, s, a);
  else if (a.head_dim == 32)
    hipLaunchKernelGGL((attn_f32_kernel<32, false>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64, false>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace hstu
