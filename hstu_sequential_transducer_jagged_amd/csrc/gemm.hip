// f1 and f2 of the HSTU layer on gfx950 MFMA ("万亿参数推荐大模型：HSTU 架构
// 如何超越传统 Self-Attention" §2.1: f1 and f2 are single linear layers).
//
//   proj: [U|V|Q|K] = SiLU(X W1^T + b1), the SiLU and the four-way split are
//         the epilogue (first equation of §2.1);
//   out:  Y = X + G W2^T + b2, bias and residual are the epilogue (third
//         equation plus the block diagram's skip connection).
//
// The same kernel, with an fp32 epilogue and optional split-K, runs the
// products of the training backward (dG, dW2, dW1, dX) on bf16 operand
// copies (launch_gemm_bf16_f32).
//
// All are C[M, N] = A[M, K] B[N, K]^T with A and B row-major and K
// contiguous, which is the operand layout of v_mfma_f32_32x32x16_bf16
// (lane = row, 8 consecutive k), so tiles are staged through LDS unchanged
// apart from a bank swizzle, by global->LDS DMA running up to three K steps
// ahead of the MFMAs.
#include <algorithm>

#include "attn_sched.h"
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Block tile: 256 rows (M) x 128 output columns (N), K staged 32 at a time.
// Four waves, each 128 rows x 64 columns; the product is formed transposed,
// C^T[n][m] = sum_k W[n][k] X[m][k] (A operand = W rows, B operand = X rows),
// so that a lane's accumulator holds 4 consecutive output columns of one row
// and the epilogue stores 8-byte bf16 quads.
//
// Operand tiles reach LDS by direct global->LDS DMA (global_load_lds_dwordx4)
// through a three-stage ring: K step s+3 is requested during step s, so each
// load has between two and three MFMA steps to land, and no staging
// registers are used. A DMA instruction writes 1 KB of consecutive LDS (16
// rows of 64 bytes); the bank swizzle is applied on the source side: the lane
// that fills 16-byte slot p of row r fetches k-chunk p ^ ((r >> 2) & 3) of
// that row, so the 16 rows one b128 MFMA-operand read serves hit 16 distinct
// bank groups.
constexpr int kGN = 128;
constexpr int kGK = 32;
constexpr int kRowB = kGK * 2;   // 64-byte LDS rows

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS byte offset of k-chunk c (0..3, 8 bf16 each) of tile row r.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ ((r >> 2) & 3)) << 4); }

// s_waitcnt immediate with vmcnt = 0 and expcnt, lgkmcnt at their maxima
// (vmcnt bits 3:0, expcnt 6:4, lgkmcnt 11:8); or in a vmcnt below 16. As a
// builtin the wait is visible to the compiler's own wait insertion.
constexpr int kWaitVm = 0x0F70;

// Workgroup barrier ordering LDS accesses only (the DMA ring is waited for
// explicitly; __syncthreads() would also drain it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Epilogues in two parts: pack() turns the 4 accumulators of row m,
// columns n..n+3 into 4 bf16 outputs (bias, activation, residual), and
// store8() writes 8 consecutive outputs of row m from column n (n % 8 == 0).
// Between them the workgroup's tile passes through LDS, so that global
// stores are whole 256-byte row segments instead of 16-byte pieces of 32
// rows per instruction.
// A pointer that is the same in every lane, held in scalar registers.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

struct ProjEpi {
  static constexpr bool kF32 = false;
  static constexpr bool kSched = true;
  const float* bias;
  uint16_t* out0;   // U, V, Q, K: the four column blocks of width K
  uint16_t* out1;
  uint16_t* out2;
  uint16_t* out3;
  int K;   // d_model: width of each of U, V, Q, K
  // the attention's work list, built by one extra workgroup when sched_nqt > 0
  // (query tiles per sequence)
  AttnArgs sched_args;
  int sched_nqt;
  __device__ __forceinline__ uint2 load_extra(int64_t, int) const { return make_uint2(0, 0); }
  // SiLU of 16 outputs (v + bias), each step over all 16 so that the
  // transcendental latencies overlap
  __device__ __forceinline__ void apply16(float (&z)[16], const uint2 (&)[4]) const {
    float t[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = __builtin_amdgcn_exp2f(-1.4426950408889634f * z[e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = __builtin_amdgcn_rcpf(1.0f + t[e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] *= t[e];
  }
  // 8 columns from n (n % 8 == 0, K % 64 == 0) lie in one block; the block
  // is picked by compares, so that the pointers stay in scalar registers
  // (readfirstlane keeps the compiler from turning the select of kernel
  // arguments into a per-lane load from the argument block). Nontemporal
  // stores: the 8 d bytes per token leave the caches to the operand tiles
  // (f1 0.24 -> 0.19 ms, the layer 2 % faster, measured on the 16 x
  // U[2048, 8192] workload).
  __device__ __forceinline__ void store8(int64_t m, int n, const uint4& o) const {
    uint16_t* p = uniform_ptr(out0);
    if (n >= K) { p = uniform_ptr(out1); n -= K; }
    if (n >= K) { p = uniform_ptr(out2); n -= K; }
    if (n >= K) { p = uniform_ptr(out3); n -= K; }
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w}, reinterpret_cast<u32x4*>(p + m * K + n));
  }
};

struct OutEpi {
  static constexpr bool kF32 = false;
  static constexpr bool kSched = false;
  const float* bias;
  const uint16_t* x;
  uint16_t* y;
  int K;
  // the residual X[m, n..n+3]
  __device__ __forceinline__ uint2 load_extra(int64_t m, int n) const {
    return *reinterpret_cast<const uint2*>(x + m * K + n);
  }
  // v + bias + X, the residual added in fp32 before the single rounding
  __device__ __forceinline__ void apply16(float (&z)[16], const uint2 (&xr)[4]) const {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      z[4 * g + 0] += bf2f(xr[g].x & 0xffff);
      z[4 * g + 1] += bf2f(xr[g].x >> 16);
      z[4 * g + 2] += bf2f(xr[g].y & 0xffff);
      z[4 * g + 3] += bf2f(xr[g].y >> 16);
    }
  }
  __device__ __forceinline__ void store8(int64_t m, int n, const uint4& o) const {
    *reinterpret_cast<uint4*>(y + m * K + n) = o;
  }
};

// fp32 output straight from the accumulators (16-byte stores of 4 columns):
// v = acc + bias (+ addend) to out, and optionally SiLU(v) split by columns
// into act[0..3] (blocks of act_w columns, row stride act_w). Split s of a
// split-K product writes to out + s * split_stride (no bias, addend or act).
struct F32Epi {
  static constexpr bool kF32 = true;
  static constexpr bool kSched = false;
  const float* bias;      // [N] or nullptr
  float* out;             // or nullptr
  const float* addend;    // or nullptr
  int64_t ld;             // row stride of out and addend
  int64_t split_stride;
  float* act[4];          // act[0] nullptr: no activation output
  int act_w;
  uint16_t* act16[4];     // bf16 copies of the act blocks, each nullptr or [M, act_w]
};

// One ring stage of DMA: wave w fills X rows 16i .. 16i+15 for i = w, w+4, ...
// (NXI instructions) and W rows for i = w, w+4 (1 KB of LDS per instruction).
template <int NXI>
__device__ __forceinline__ void gemm_issue(const uint16_t* const* xsrc, const uint16_t* const* wsrc,
                                           uint8_t* sx, uint8_t* sw, int k0, int wave) {
#pragma unroll
  for (int i = 0; i < NXI; ++i)
    __builtin_amdgcn_global_load_lds(xsrc[i] + k0, LDS_PTR(void, sx + (wave + 4 * i) * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds(wsrc[i] + k0, LDS_PTR(void, sw + (wave + 4 * i) * 1024), 16, 0, 0);
}

// LDS operand reads of one 16-deep half (kk) of a 32-deep K stage.
template <int NJ>
__device__ __forceinline__ void gemm_ops(const uint8_t* sx, const uint8_t* sw, int kk, bf16x8 (&a)[2],
                                         bf16x8 (&b)[NJ], int wm, int wn, int l32, int h) {
  const int c = 2 * kk + h;          // 16-byte chunk of this lane's 8 k values
#pragma unroll
  for (int i = 0; i < 2; ++i)
    a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sw[swz(wn * 64 + i * 32 + l32, c)]));
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sx[swz(wm * 32 * NJ + j * 32 + l32, c)]));
}

template <int NJ>
__device__ __forceinline__ void gemm_mma(const bf16x8 (&a)[2], const bf16x8 (&b)[NJ], f32x16 (&acc)[2][NJ]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
}

// The K loop over the three-stage ring, with two operand register sets.
// Step s: read the second half of stage s (set 1), multiply the first half
// (set 0, read during step s-1); wait for this wave's DMA of stage s+1 and
// barrier (stage s+1 is in LDS for every wave, and every wave has read all of
// stage s); request stage s+3 into stage s's buffer; read the first half of
// stage s+1 (set 0); multiply set 1. LDS reads thus overlap the MFMAs of the
// other set, and each DMA has between two and three steps to land. The stage
// buffers are separate LDS arrays, passed as distinct restrict-qualified
// pointers, so the compiler's own waits leave the DMA in flight while other
// stages are read.
template <int NJ, int NSTEPS>
__device__ __forceinline__ void gemm_mainloop(uint8_t* __restrict__ sX0, uint8_t* __restrict__ sX1,
                                              uint8_t* __restrict__ sX2, uint8_t* __restrict__ sW0,
                                              uint8_t* __restrict__ sW1, uint8_t* __restrict__ sW2,
                                              const uint16_t* const (&xsrc)[NJ],
                                              const uint16_t* const (&wsrc)[2], f32x16 (&acc)[2][NJ],
                                              int nsteps_rt, int wave, int wm, int wn, int l32, int h) {
  const int nsteps = NSTEPS > 0 ? NSTEPS : nsteps_rt;
  gemm_issue<NJ>(xsrc, wsrc, sX0, sW0, 0, wave);
  if (nsteps > 1) gemm_issue<NJ>(xsrc, wsrc, sX1, sW1, kGK, wave);
  if (nsteps > 2) gemm_issue<NJ>(xsrc, wsrc, sX2, sW2, 2 * kGK, wave);
  if (nsteps > 2)
    __builtin_amdgcn_s_waitcnt(kWaitVm | (2 * (NJ + 2)));
  else if (nsteps > 1)
    __builtin_amdgcn_s_waitcnt(kWaitVm | (NJ + 2));
  else
    __builtin_amdgcn_s_waitcnt(kWaitVm);
  lds_barrier();
  bf16x8 a0[2], b0[NJ], a1[2], b1[NJ];
  gemm_ops<NJ>(sX0, sW0, 0, a0, b0, wm, wn, l32, h);
  // (scheduling fences keep each set's LDS reads ahead of the other set's
  // MFMAs; left alone, the compiler sinks the reads to just before their use)
#define HSTU_GEMM_STEP(s, CX, CW, NX, NW)                                      \
  {                                                                            \
    gemm_ops<NJ>(CX, CW, 1, a1, b1, wm, wn, l32, h);                           \
    __builtin_amdgcn_sched_barrier(0);                                         \
    gemm_mma<NJ>(a0, b0, acc);                                                 \
    if ((s) + 1 < nsteps) {                                                    \
      if ((s) + 2 < nsteps)                                                    \
        __builtin_amdgcn_s_waitcnt(kWaitVm | (NJ + 2));                        \
      else                                                                     \
        __builtin_amdgcn_s_waitcnt(kWaitVm);                                   \
      lds_barrier();                                                           \
      if ((s) + 3 < nsteps) gemm_issue<NJ>(xsrc, wsrc, CX, CW, ((s) + 3) * kGK, wave); \
      gemm_ops<NJ>(NX, NW, 0, a0, b0, wm, wn, l32, h);                         \
    }                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                         \
    gemm_mma<NJ>(a1, b1, acc);                                                 \
  }
  int s = 0;
#pragma unroll
  for (; s + 3 <= nsteps; s += 3) {
    HSTU_GEMM_STEP(s, sX0, sW0, sX1, sW1)
    HSTU_GEMM_STEP(s + 1, sX1, sW1, sX2, sW2)
    HSTU_GEMM_STEP(s + 2, sX2, sW2, sX0, sW0)
  }
  if (s < nsteps) {
    HSTU_GEMM_STEP(s, sX0, sW0, sX1, sW1)
    if (s + 1 < nsteps) HSTU_GEMM_STEP(s + 1, sX1, sW1, sX2, sW2)
  }
#undef HSTU_GEMM_STEP
}

// The output tile after the K loop: BM rows of 128 bf16 (256 B), in 32-row
// blocks of 8 KB laid over the ring arrays (NJ/2 blocks per X stage, one per
// W stage). The 16-byte chunk c of row r sits at chunk c ^ (r & 15), so that
// the 32 rows one accumulator store covers spread over the banks.
template <int NJ>
__device__ __forceinline__ uint8_t* tile_block(int b, uint8_t* sX0, uint8_t* sX1, uint8_t* sX2,
                                               uint8_t* sW0, uint8_t* sW1, uint8_t* sW2) {
  constexpr int XB = NJ / 2;
  if (b < XB) return sX0 + b * 8192;
  if (b < 2 * XB) return sX1 + (b - XB) * 8192;
  if (b < 3 * XB) return sX2 + (b - 2 * XB) * 8192;
  if (b == 3 * XB) return sW0;
  if (b == 3 * XB + 1) return sW1;
  return sW2;
}

__device__ __forceinline__ int tile_off(int r, int c) { return (r & 31) * 256 + ((c ^ (r & 15)) << 4); }

// X [M, ldx] row-major, W [N, ldw] row-major (nn.Linear), contracted over
// K columns (K % 32 == 0), N % 4 == 0. Grid, with splits == 1:
// 8 * ceil(nm / 8) * nn workgroups (nm = ceil(M/BM), nn = ceil(N/128));
// workgroup id -> XCD id % 8 (round-robin dispatch); XCD x takes row blocks
// x, x+8, ... and sweeps all nn column tiles of one row block before the
// next, so each X row block is read from HBM once and W stays in that XCD's
// L2. With splits > 1 (split-K, few tiles): splits * nm * nn workgroups,
// tile-major within a split; split s contracts columns s*K .. s*K + K - 1.
template <int NJ, class Epi>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W,
                                                           int64_t M, int N, int K, int64_t ldx,
                                                           int64_t ldw, int nm, int nn, int splits,
                                                           Epi epi) {
  constexpr int BM = 64 * NJ;      // block rows; each wave owns BM/2 rows x 64 columns
  // The three ring stages are separate LDS arrays: the compiler's wait
  // insertion tells DMA into one array apart from reads of another only for
  // distinct arrays, and would otherwise wait for every DMA in flight before
  // each stage's first read. After the K loop the same arrays hold the
  // output tile (tile_block).
  __shared__ __attribute__((aligned(16))) uint8_t sX0[BM * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t sX1[BM * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t sX2[BM * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t sW0[kGN * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t sW1[kGN * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t sW2[kGN * kRowB];
  __shared__ __attribute__((aligned(16))) float sbias[kGN];   // bias of the tile's columns (0 past N)
  static_assert(3 * BM * kRowB + 3 * kGN * kRowB >= BM * 256, "output tile must fit the ring");
  if constexpr (Epi::kSched) {
    // the extra last workgroup builds the following attention's work list,
    // with the first ring stage as its counters and the bias slots as its
    // scan slots
    static_assert(BM * kRowB >= sched::kListInts * 4 && kGN * 4 >= 4 * 8, "work-list scratch");
    if (epi.sched_nqt > 0 && blockIdx.x == gridDim.x - 1) {
      sched::build<256>(epi.sched_args, epi.sched_nqt, reinterpret_cast<int*>(sX0),
                        reinterpret_cast<long long*>(sbias));
      return;
    }
  }

  const int id = blockIdx.x;
  int mb, nb, sp = 0;
  if (splits == 1) {
    const int xcd = id & 7;
    const int slot = id >> 3;
    mb = (slot / nn) * 8 + xcd;
    nb = slot - (slot / nn) * nn;
    if (mb >= nm) return;
  } else {
    const int nt = nm * nn;
    sp = id / nt;
    const int t = id - sp * nt;
    mb = t / nn;
    nb = t - mb * nn;
  }
  const int64_t m0 = static_cast<int64_t>(mb) * BM;
  const int n0 = nb * kGN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave & 1;         // row half
  const int wn = wave >> 1;        // 64-column half
  const int l32 = lane & 31;
  const int h = lane >> 5;
  if (tid < kGN) sbias[tid] = (epi.bias && n0 + tid < N) ? epi.bias[n0 + tid] : 0.0f;

  // DMA source rows of this lane: X instructions cover rows 16i + lane/4
  // (i = wave, wave+4, ...), W instructions rows 16i + lane/4 (i = wave,
  // wave+4). Rows past M or N repeat the last valid row: their products land
  // only in outputs that are not stored.
  const int lr = lane >> 2;
  const int lp = lane & 3;
  const uint16_t* xsrc[NJ];
  const uint16_t* wsrc[2];
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int r = 16 * (wave + 4 * i) + lr;
    const int64_t gm = min(m0 + r, M - 1);
    xsrc[i] = X + gm * ldx + static_cast<int64_t>(sp) * K + 8 * (lp ^ ((r >> 2) & 3));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (wave + 4 * i) + lr;
    const int gn = min(n0 + r, N - 1);
    wsrc[i] = W + gn * ldw + static_cast<int64_t>(sp) * K + 8 * (lp ^ ((r >> 2) & 3));
  }
  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  switch (K / kGK) {   // common widths (d_model 256, 512, 1024): unrolled
    case 8: gemm_mainloop<NJ, 8>(sX0, sX1, sX2, sW0, sW1, sW2, xsrc, wsrc, acc, 8, wave, wm, wn, l32, h); break;
    case 16: gemm_mainloop<NJ, 16>(sX0, sX1, sX2, sW0, sW1, sW2, xsrc, wsrc, acc, 16, wave, wm, wn, l32, h); break;
    case 32: gemm_mainloop<NJ, 32>(sX0, sX1, sX2, sW0, sW1, sW2, xsrc, wsrc, acc, 32, wave, wm, wn, l32, h); break;
    default: gemm_mainloop<NJ, 0>(sX0, sX1, sX2, sW0, sW1, sW2, xsrc, wsrc, acc, K / kGK, wave, wm, wn, l32, h);
  }

  if constexpr (Epi::kF32) {
    // C^T accumulator: lane -> row j*32 + lane%32, columns
    // i*32 + 8*(r/4) + 4*h + r%4 of the wave's block
    float* const out = epi.out ? epi.out + sp * epi.split_stride : nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t m = m0 + wm * 32 * NJ + j * 32 + l32;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * 64 + i * 32 + 8 * g + 4 * h;
          const int n = n0 + nl;
          if (m < M && n < N) {
            const float4 b = *reinterpret_cast<const float4*>(&sbias[nl]);
            float4 v = make_float4(acc[i][j][4 * g + 0] + b.x, acc[i][j][4 * g + 1] + b.y,
                                   acc[i][j][4 * g + 2] + b.z, acc[i][j][4 * g + 3] + b.w);
            if (epi.addend) {
              const float4 r = *reinterpret_cast<const float4*>(epi.addend + m * epi.ld + n);
              v.x += r.x;
              v.y += r.y;
              v.z += r.z;
              v.w += r.w;
            }
            if (out) *reinterpret_cast<float4*>(out + m * epi.ld + n) = v;
            if (epi.act[0]) {
              // the 4 columns lie in one block (act_w % 4 == 0)
              int c = n;
              float* p = epi.act[0];
              uint16_t* p16 = epi.act16[0];
              if (c >= epi.act_w) { p = epi.act[1]; p16 = epi.act16[1]; c -= epi.act_w; }
              if (c >= epi.act_w) { p = epi.act[2]; p16 = epi.act16[2]; c -= epi.act_w; }
              if (c >= epi.act_w) { p = epi.act[3]; p16 = epi.act16[3]; c -= epi.act_w; }
              float4 a;
              a.x = v.x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v.x));
              a.y = v.y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v.y));
              a.z = v.z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v.z));
              a.w = v.w * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v.w));
              *reinterpret_cast<float4*>(p + m * epi.act_w + c) = a;
              if (p16)
                *reinterpret_cast<uint2*>(p16 + m * epi.act_w + c) =
                    make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
            }
          }
        }
    }
  } else {
  // Output tile through LDS. C^T accumulator: lane -> row j*32 + lane%32,
  // columns i*32 + 8*(r/4) + 4*h + r%4 of the wave's block.
  // Per-element epilogue inputs (the residual of f2) are loaded first, all
  // at once and unconditionally (rows and columns clamped), so that their
  // latencies overlap; loads behind a bounds branch would each be waited
  // for on their own.
  uint2 extra[NJ][2][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t m = min(m0 + wm * 32 * NJ + j * 32 + l32, M - 1);
        const int n = min(n0 + wn * 64 + i * 32 + 8 * g + 4 * h, N - 4);
        extra[j][i][g] = epi.load_extra(m, n);
      }
  lds_barrier();   // every wave is done reading the ring
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ml = wm * 32 * NJ + j * 32 + l32;
    const int64_t m = m0 + ml;
    uint8_t* const blk = tile_block<NJ>(wm * NJ + j, sX0, sX1, sX2, sW0, sW1, sW2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float z[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 b = *reinterpret_cast<const float4*>(&sbias[wn * 64 + i * 32 + 8 * g + 4 * h]);
        z[4 * g + 0] = acc[i][j][4 * g + 0] + b.x;
        z[4 * g + 1] = acc[i][j][4 * g + 1] + b.y;
        z[4 * g + 2] = acc[i][j][4 * g + 2] + b.z;
        z[4 * g + 3] = acc[i][j][4 * g + 3] + b.w;
      }
      epi.apply16(z, extra[j][i]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * 64 + i * 32 + 8 * g + 4 * h;
        const uint2 o = make_uint2(pack_bf16x2(z[4 * g + 0], z[4 * g + 1]),
                                   pack_bf16x2(z[4 * g + 2], z[4 * g + 3]));
        *reinterpret_cast<uint2*>(blk + tile_off(ml, nl >> 3) + 8 * h) =
            (m < M && n0 + nl < N) ? o : make_uint2(0, 0);
      }
    }
  }
  lds_barrier();
  // 16 threads per 256-byte row segment, 16 rows per pass
#pragma unroll
  for (int it = 0; it < BM / 16; ++it) {
    const int row = it * 16 + (tid >> 4);
    const int nl = (tid & 15) * 8;
    const int64_t m = m0 + row;
    const uint8_t* const blk = tile_block<NJ>(it / 2, sX0, sX1, sX2, sW0, sW1, sW2);
    if (m < M && n0 + nl < N)
      epi.store8(m, n0 + nl, *reinterpret_cast<const uint4*>(blk + tile_off(row, tid & 15)));
  }
  }
}

// ---------------------------------------------------------------------------
// fp32: 16 x 16 output tile per block, K staged through LDS in steps of 16.
// Used where the matrix-core kernel (gemm_f32.hip) refuses the layout.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B, int64_t M,
                                                       int N, int K, Epi epi) {
  __shared__ float sA[16][17];
  __shared__ float sB[16][17];
  const int tx = threadIdx.x & 15;
  const int ty = threadIdx.x >> 4;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 16 + ty;
  const int n = blockIdx.y * 16 + tx;
  float acc = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int64_t am = static_cast<int64_t>(blockIdx.x) * 16 + ty;
    const int bn = blockIdx.y * 16 + ty;
    sA[ty][tx] = (am < M && k0 + tx < K) ? A[am * K + k0 + tx] : 0.0f;
    sB[ty][tx] = (bn < N && k0 + tx < K) ? B[static_cast<int64_t>(bn) * K + k0 + tx] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sA[ty][kk], sB[tx][kk], acc);
    __syncthreads();
  }
  if (m < M && n < N) epi(m, n, acc);
}

struct ProjEpiF32 {
  const float* bias;
  float* out[4];
  int K;
  __device__ __forceinline__ void operator()(int64_t m, int n, float acc) const {
    const float z = acc + (bias ? bias[n] : 0.0f);
    const int chunk = n / K;
    out[chunk][m * K + (n - chunk * K)] = z / (1.0f + expf(-z));
  }
};

struct OutEpiF32 {
  const float* bias;
  const float* x;
  float* y;
  int K;
  __device__ __forceinline__ void operator()(int64_t m, int n, float acc) const {
    y[m * K + n] = acc + (bias ? bias[n] : 0.0f) + x[m * K + n];
  }
};

}  // namespace

// 256-row blocks (measured faster on long inputs), or 128-row blocks when
// 256-row ones would give the 512 workgroup slots (two per compute unit)
// under four rounds of work: f2 of the 16 x U[2048, 8192] layer (1 204
// tiles of 256 rows) runs 128-row tiles, and the whole layer is 2 % faster
// so (measured in both launch orders), although f2 alone is 4 us slower.
template <class Epi>
hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int N, int K, Epi epi,
                            hipStream_t s) {
  const int nn = (N + kGN - 1) / kGN;
  const int64_t blocks256 = (M + 255) / 256 * nn;
  int extra = 0;   // the work-list workgroup
  if constexpr (Epi::kSched) extra = epi.sched_nqt > 0 ? 1 : 0;
  if (blocks256 >= 4 * 512) {
    const int nm = static_cast<int>((M + 255) / 256);
    const int grid = 8 * ((nm + 7) / 8) * nn + extra;
    hipLaunchKernelGGL((gemm_bf16_kernel<4, Epi>), dim3(grid), dim3(256), 0, s, x, w, M, N, K,
                       static_cast<int64_t>(K), static_cast<int64_t>(K), nm, nn, 1, epi);
  } else {
    const int nm = static_cast<int>((M + 127) / 128);
    const int grid = 8 * ((nm + 7) / 8) * nn + extra;
    hipLaunchKernelGGL((gemm_bf16_kernel<2, Epi>), dim3(grid), dim3(256), 0, s, x, w, M, N, K,
                       static_cast<int64_t>(K), static_cast<int64_t>(K), nm, nn, 1, epi);
  }
  return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void sum_splits_kernel(const float4* __restrict__ part, int splits,
                                                         int64_t n4, float4* __restrict__ out) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float4 a = part[i];
    for (int sp = 1; sp < splits; ++sp) {
      const float4 b = part[sp * n4 + i];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    out[i] = a;
  }
}

// 64 x 64 tiles: coalesced float4 row reads into LDS, then 16-byte bf16
// writes of the transposed rows (8 consecutive source rows per thread). The
// 65-float LDS rows make both the stores and the column reads conflict-free.
// With dst_rows the same rounded values also go out untransposed (row
// stride ld_rows), from the row reads; with rows_x3 as the hi/lo split rows
// [hi | lo | hi] of to_bf16x3_kernel below (lo_last = 0). With colsum, the
// tile's fp32 column sums are added to colsum[c] atomically. S: fp32 source,
// or bf16 (raw 16-bit patterns; the copies are then exact).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf2f(w.x & 0xffff), bf2f(w.x >> 16), bf2f(w.y & 0xffff), bf2f(w.y >> 16));
}
template <typename S>
__global__ __launch_bounds__(256) void to_bf16_t_kernel(const S* __restrict__ src, int64_t ld_src,
                                                        int64_t rows, int cols, uint16_t* __restrict__ dst,
                                                        int64_t ld_dst, uint16_t* __restrict__ dst_rows,
                                                        int64_t ld_rows, int rows_x3, float* colsum) {
  __shared__ float t[64][65];
  __shared__ float part[4][64];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * 16 + (tid >> 4);
    const int c = (tid & 15) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + r < rows && c0 + c < cols) {
      v = load4(src + (r0 + r) * ld_src + c0 + c);
      if (dst_rows) {
        uint16_t* const o = dst_rows + (r0 + r) * ld_rows + c0 + c;
        const uint2 hi = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        *reinterpret_cast<uint2*>(o) = hi;
        if (rows_x3) {
          const float4 l = make_float4(v.x - bf2f(hi.x & 0xffff), v.y - bf2f(hi.x >> 16),
                                       v.z - bf2f(hi.y & 0xffff), v.w - bf2f(hi.y >> 16));
          *reinterpret_cast<uint2*>(o + cols) = make_uint2(pack_bf16x2(l.x, l.y), pack_bf16x2(l.z, l.w));
          *reinterpret_cast<uint2*>(o + 2 * cols) = hi;
        }
      }
    }
    t[r][c + 0] = v.x;
    t[r][c + 1] = v.y;
    t[r][c + 2] = v.z;
    t[r][c + 3] = v.w;
  }
  __syncthreads();
  if (colsum) {
    // four quarters of 16 rows per column, then one atomic per column
    const int cc = tid & 63, q = tid >> 6;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += t[16 * q + r][cc];
    part[q][cc] = sum;
    __syncthreads();
    if (tid < 64 && c0 + tid < cols && r0 < rows)
      atomicAdd(&colsum[c0 + tid], (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]));
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = it * 256 + tid;
    const int cc = idx >> 3;
    const int ch = idx & 7;
    if (c0 + cc < cols && r0 + ch * 8 < ld_dst) {
      uint4 o;
      o.x = pack_bf16x2(t[ch * 8 + 0][cc], t[ch * 8 + 1][cc]);
      o.y = pack_bf16x2(t[ch * 8 + 2][cc], t[ch * 8 + 3][cc]);
      o.z = pack_bf16x2(t[ch * 8 + 4][cc], t[ch * 8 + 5][cc]);
      o.w = pack_bf16x2(t[ch * 8 + 6][cc], t[ch * 8 + 7][cc]);
      *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(c0 + cc) * ld_dst + r0 + ch * 8) = o;
    }
  }
}

// Row r of src (cols floats) -> row r of dst (3 cols bf16): x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi); the three column blocks are
// [hi | lo | hi] (lo_last == 0) or [hi | hi | lo] (lo_last == 1), so that
// [A_hi | A_lo | A_hi] [B_hi | B_hi | B_lo]^T = A_hi B_hi^T + A_lo B_hi^T +
// A_hi B_lo^T: the product of the two fp32 matrices up to the lo*lo term.
__global__ __launch_bounds__(256) void to_bf16x3_kernel(const float4* __restrict__ src, int64_t rows, int cols4,
                                                        uint2* __restrict__ dst, int lo_last) {
  const int64_t n4 = rows * cols4;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cols4;
    const int64_t c = i - r * cols4;
    const float4 v = src[i];
    const uint2 hi = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    const float4 l = make_float4(v.x - bf2f(hi.x & 0xffff), v.y - bf2f(hi.x >> 16), v.z - bf2f(hi.y & 0xffff),
                                 v.w - bf2f(hi.y >> 16));
    const uint2 lo = make_uint2(pack_bf16x2(l.x, l.y), pack_bf16x2(l.z, l.w));
    uint2* const row = dst + r * 3 * cols4;
    row[c] = hi;
    row[cols4 + c] = lo_last ? hi : lo;
    row[2 * cols4 + c] = lo_last ? lo : hi;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_to_bf16x3(const float* src, int64_t rows, int cols, uint16_t* dst, int lo_last, hipStream_t s) {
  if (cols % 4 != 0 || !aligned16(src) || !aligned16(dst)) return hipErrorInvalidValue;
  const int64_t n4 = rows * (cols / 4);
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(to_bf16x3_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(src), rows, cols / 4, reinterpret_cast<uint2*>(dst), lo_last);
  return hipGetLastError();
}

// Split-K products (the weight gradients, few output tiles) take 256-row
// blocks from M = 2048 up; single products the forward's rule.
hipError_t launch_gemm_bf16_f32(const GemmBf16Args& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const bool act = g.act[0] != nullptr;
  if (g.kc <= 0 || g.kc % kGK != 0 || g.splits < 1 || g.lda % 8 != 0 || g.ldb % 8 != 0 || g.N % 4 != 0 ||
      g.ldc % 4 != 0 || g.ldc < g.N || g.lda < static_cast<int64_t>(g.splits) * g.kc ||
      g.ldb < static_cast<int64_t>(g.splits) * g.kc ||
      (g.splits > 1 && (g.addend || g.bias || act || !g.c)) || !aligned16(g.a) || !aligned16(g.b) ||
      (g.c && !aligned16(g.c)) || (g.addend && !aligned16(g.addend)) ||
      (act && (g.act_w <= 0 || g.act_w % 4 != 0 || static_cast<int64_t>(g.act_w) * 4 != g.N)))
    return hipErrorInvalidValue;
  for (int i = 0; i < 4; ++i)
    if ((act && (!g.act[i] || !aligned16(g.act[i]))) || (g.act16[i] && (!act || !aligned16(g.act16[i]))))
      return hipErrorInvalidValue;
  const F32Epi epi{g.bias, g.c, g.addend, g.ldc, g.M * g.ldc, {g.act[0], g.act[1], g.act[2], g.act[3]},
                   g.act_w, {g.act16[0], g.act16[1], g.act16[2], g.act16[3]}};
  const int nn = (g.N + kGN - 1) / kGN;
  const bool big = g.splits > 1 ? g.M >= 2048 : (g.M + 255) / 256 * nn >= 2 * 512;
  const int bm = big ? 256 : 128;
  const int64_t nm = (g.M + bm - 1) / bm;
  const int64_t grid = g.splits > 1 ? g.splits * nm * nn : 8 * ((nm + 7) / 8) * nn;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (big)
    hipLaunchKernelGGL((gemm_bf16_kernel<4, F32Epi>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, g.a,
                       g.b, g.M, g.N, g.kc, g.lda, g.ldb, static_cast<int>(nm), nn, g.splits, epi);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<2, F32Epi>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, g.a,
                       g.b, g.M, g.N, g.kc, g.lda, g.ldb, static_cast<int>(nm), nn, g.splits, epi);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int splits, int64_t n, float* out, hipStream_t s) {
  if (n % 4 != 0 || splits < 1 || !aligned16(part) || !aligned16(out)) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(sum_splits_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(part), splits, n4, reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

hipError_t launch_to_bf16_t(const float* src, int64_t ld_src, int64_t rows, int cols, uint16_t* dst,
                            int64_t ld_dst, hipStream_t s, uint16_t* dst_rows, int64_t ld_rows, bool rows_x3,
                            float* colsum) {
  if (cols % 4 != 0 || ld_src % 4 != 0 || ld_src < cols || ld_dst % 8 != 0 || ld_dst < rows || !aligned16(src) ||
      !aligned16(dst))
    return hipErrorInvalidValue;
  if (dst_rows && (ld_rows % 4 != 0 || ld_rows < (rows_x3 ? 3 : 1) * static_cast<int64_t>(cols) ||
                   (reinterpret_cast<uintptr_t>(dst_rows) & 7u) != 0))
    return hipErrorInvalidValue;
  if (cols == 0 || ld_dst == 0) return hipSuccess;
  const int64_t gx = (ld_dst + 63) / 64;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(to_bf16_t_kernel<float>, dim3(static_cast<unsigned>(gx), (cols + 63) / 64), dim3(256), 0, s,
                     src, ld_src, rows, cols, dst, ld_dst, dst_rows, ld_rows, rows_x3 ? 1 : 0, colsum);
  return hipGetLastError();
}

hipError_t launch_bf16_t(const uint16_t* src, int64_t ld_src, int64_t rows, int cols, uint16_t* dst,
                         int64_t ld_dst, hipStream_t s) {
  if (cols % 4 != 0 || ld_src % 4 != 0 || ld_src < cols || ld_dst % 8 != 0 || ld_dst < rows ||
      (reinterpret_cast<uintptr_t>(src) & 7u) != 0 || !aligned16(dst))
    return hipErrorInvalidValue;
  if (cols == 0 || ld_dst == 0) return hipSuccess;
  const int64_t gx = (ld_dst + 63) / 64;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(to_bf16_t_kernel<uint16_t>, dim3(static_cast<unsigned>(gx), (cols + 63) / 64), dim3(256), 0,
                     s, src, ld_src, rows, cols, dst, ld_dst, nullptr, 0, 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_proj_bf16(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  ProjEpi epi{};
  epi.bias = a.bias;
  epi.out0 = static_cast<uint16_t*>(a.out[0]);
  epi.out1 = static_cast<uint16_t*>(a.out[1]);
  epi.out2 = static_cast<uint16_t*>(a.out[2]);
  epi.out3 = static_cast<uint16_t*>(a.out[3]);
  epi.K = a.K;
  if (a.sched && a.sched->num_seqs > 0 && a.sched->max_seq_len > 0) {
    if (a.sched->bm != kAttnBM) return hipErrorInvalidValue;
    epi.sched_args = *a.sched;
    epi.sched_nqt = (a.sched->max_seq_len + kAttnBM - 1) / kAttnBM;
  }
  return launch_gemm_bf16(static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.w), a.M,
                          4 * a.K, a.K, epi, s);
}

hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  OutEpi epi{a.bias, static_cast<const uint16_t*>(a.x), static_cast<uint16_t*>(a.y), a.K};
  return launch_gemm_bf16(static_cast<const uint16_t*>(a.g), static_cast<const uint16_t*>(a.w), a.M,
                          a.K, a.K, epi, s);
}

hipError_t launch_proj_f32(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const int N = 4 * a.K;
  if (a.M < (int64_t{1} << 31)) {
    GemmF32Args g{};
    g.A = static_cast<const float*>(a.x); g.sam = a.K; g.sak = 1;
    g.B = static_cast<const float*>(a.w); g.sbk = 1; g.sbn = a.K;
    g.bias = a.bias;
    for (int i = 0; i < 4; ++i) g.outs[i] = static_cast<float*>(a.out[i]);
    g.split = a.K; g.M = static_cast<int>(a.M); g.N = N; g.K = a.K;
    const hipError_t e = launch_gemm_f32_mma(g, 2, 1, s);
    if (e != hipErrorNotSupported) return e;
  }
  ProjEpiF32 epi{a.bias,
                 {static_cast<float*>(a.out[0]), static_cast<float*>(a.out[1]),
                  static_cast<float*>(a.out[2]), static_cast<float*>(a.out[3])},
                 a.K};
  dim3 grid(static_cast<unsigned>((a.M + 15) / 16), (N + 15) / 16);
  hipLaunchKernelGGL(gemm_f32_kernel<ProjEpiF32>, grid, dim3(256), 0, s,
                     static_cast<const float*>(a.x), static_cast<const float*>(a.w), a.M, N,
                     a.K, epi);
  return hipGetLastError();
}

hipError_t launch_out_f32(const OutArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.M < (int64_t{1} << 31)) {
    GemmF32Args g{};
    g.A = static_cast<const float*>(a.g); g.sam = a.K; g.sak = 1;
    g.B = static_cast<const float*>(a.w); g.sbk = 1; g.sbn = a.K;
    g.C = static_cast<float*>(a.y); g.ldc = a.K;
    g.addend = static_cast<const float*>(a.x); g.bias = a.bias;
    g.M = static_cast<int>(a.M); g.N = a.K; g.K = a.K;
    const hipError_t e = launch_gemm_f32_mma(g, 0, 1, s);
    if (e != hipErrorNotSupported) return e;
  }
  OutEpiF32 epi{a.bias, static_cast<const float*>(a.x), static_cast<float*>(a.y), a.K};
  dim3 grid(static_cast<unsigned>((a.M + 15) / 16), (a.K + 15) / 16);
  hipLaunchKernelGGL(gemm_f32_kernel<OutEpiF32>, grid, dim3(256), 0, s,
                     static_cast<const float*>(a.g), static_cast<const float*>(a.w), a.M, a.K,
                     a.K, epi);
  return hipGetLastError();
}

}  // namespace hstu
