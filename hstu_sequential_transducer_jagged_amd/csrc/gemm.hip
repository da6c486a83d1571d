// f1 and f2 of the HSTU layer on gfx950 MFMA ("万亿参数推荐大模型：HSTU 架构
// 如何超越传统 Self-Attention" §2.1: f1 and f2 are single linear layers).
//
//   proj: [U|V|Q|K] = SiLU(X W1^T + b1), the SiLU and the four-way split are
//         the epilogue (first equation of §2.1);
//   out:  Y = X + G W2^T + b2, bias and residual are the epilogue (third
//         equation plus the block diagram's skip connection).
//
// Both are C[M, N] = A[M, K] B[N, K]^T with A and B row-major and K
// contiguous, which is the operand layout of v_mfma_f32_32x32x16_bf16
// (lane = row, 8 consecutive k), so tiles are staged through LDS unchanged
// apart from a bank swizzle. The next K step's global loads are issued
// before the current step's MFMAs (register staging, double-buffered LDS).
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Block tile: 256 rows (M) x 128 output columns (N), K staged 32 at a time.
// Four waves, each 128 rows x 64 columns; the product is formed transposed,
// C^T[n][m] = sum_k W[n][k] X[m][k] (A operand = W rows, B operand = X rows),
// so that a lane's accumulator holds 4 consecutive output columns of one row
// and the epilogue stores 8-byte bf16 quads.
//
// Operand tiles reach LDS by direct global->LDS DMA (global_load_lds_dwordx4)
// through a three-stage ring: the K step s+2 is requested while step s is
// multiplied, so each load has two MFMA steps to land, and no staging
// registers are used. A DMA instruction writes 1 KB of consecutive LDS (16
// rows of 64 bytes); the bank swizzle is applied on the source side: the lane
// that fills 16-byte slot p of row r fetches k-chunk p ^ ((r >> 2) & 3) of
// that row, so the 16 rows one b128 MFMA-operand read serves hit 16 distinct
// bank groups.
constexpr int kGN = 128;
constexpr int kGK = 32;
constexpr int kRowB = kGK * 2;   // 64-byte LDS rows
constexpr int kOutRowB = kGN * 2 + 8;   // output tile row: 128 bf16 + 8-byte pad (conflict-free)

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS byte offset of k-chunk c (0..3, 8 bf16 each) of tile row r.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

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
struct ProjEpi {
  const float* bias;
  uint16_t* out[4];
  int K;   // d_model: width of each of U, V, Q, K
  __device__ __forceinline__ uint2 pack(int64_t, int, const float (&v)[4], const float4& b) const {
    const float bb[4] = {b.x, b.y, b.z, b.w};
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = silu_fast(v[e] + bb[e]);
    return make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
  }
  __device__ __forceinline__ void store8(int64_t m, int n, const uint4& o) const {
    const int chunk = n / K;
    *reinterpret_cast<uint4*>(out[chunk] + m * K + (n - chunk * K)) = o;
  }
};

struct OutEpi {
  const float* bias;
  const uint16_t* x;
  uint16_t* y;
  int K;
  __device__ __forceinline__ uint2 pack(int64_t m, int n, const float (&v)[4], const float4& b) const {
    const uint2 xr = *reinterpret_cast<const uint2*>(x + m * K + n);
    const float xv[4] = {bf2f(xr.x & 0xffff), bf2f(xr.x >> 16), bf2f(xr.y & 0xffff), bf2f(xr.y >> 16)};
    const float bb[4] = {b.x, b.y, b.z, b.w};
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = v[e] + bb[e] + xv[e];
    return make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
  }
  __device__ __forceinline__ void store8(int64_t m, int n, const uint4& o) const {
    *reinterpret_cast<uint4*>(y + m * K + n) = o;
  }
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

// One 32-deep K step of a wave's (32 NJ) x 64 tile (C^T: 64 x 32 NJ).
template <int NJ>
__device__ __forceinline__ void gemm_compute(const uint8_t* sx, const uint8_t* sw, f32x16 (&acc)[2][NJ],
                                             int wm, int wn, int l32, int h) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {     // two 16-deep MFMA steps
    const int c = 2 * kk + h;          // 16-byte chunk of this lane's 8 k values
    bf16x8 a[2], b[NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sw[swz(wn * 64 + i * 32 + l32, c)]));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sx[swz(wm * 32 * NJ + j * 32 + l32, c)]));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

// The K loop over the three-stage ring. The stage buffers come in as
// __restrict__ pointers: once inlined, every LDS access and DMA carries alias
// scopes that tell the compiler's wait insertion that a DMA into one stage
// does not alias reads of another, so it waits only for the stage it reads.
// Step s: wait for this wave's DMA of stage s (the NJ + 2 instructions of
// stage s+1 may stay in flight), barrier so that every wave's stage s is in LDS and
// every wave is done with stage s-1, request stage s+2 into the buffer of
// stage s-1, multiply stage s.
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
#define HSTU_GEMM_STEP(s, SX, SW, NX, NW)                                      \
  {                                                                            \
    if ((s) + 1 < nsteps)                                                      \
      __builtin_amdgcn_s_waitcnt(kWaitVm | (NJ + 2));                          \
    else                                                                       \
      __builtin_amdgcn_s_waitcnt(kWaitVm);                                     \
    lds_barrier();                                                             \
    if ((s) + 2 < nsteps) gemm_issue<NJ>(xsrc, wsrc, NX, NW, ((s) + 2) * kGK, wave); \
    gemm_compute<NJ>(SX, SW, acc, wm, wn, l32, h);                             \
  }
  int s = 0;
#pragma unroll
  for (; s + 3 <= nsteps; s += 3) {
    HSTU_GEMM_STEP(s, sX0, sW0, sX2, sW2)
    HSTU_GEMM_STEP(s + 1, sX1, sW1, sX0, sW0)
    HSTU_GEMM_STEP(s + 2, sX2, sW2, sX1, sW1)
  }
  if (s < nsteps) {
    HSTU_GEMM_STEP(s, sX0, sW0, sX2, sW2)
    if (s + 1 < nsteps) HSTU_GEMM_STEP(s + 1, sX1, sW1, sX0, sW0)
  }
#undef HSTU_GEMM_STEP
}

// X [M, K] row-major, W [N, K] row-major (nn.Linear), K % 32 == 0,
// N % 4 == 0. Grid: 8 * ceil(nm / 8) * nn workgroups (nm = ceil(M/256),
// nn = ceil(N/128)); workgroup id -> XCD id % 8 (round-robin dispatch); XCD x
// takes row blocks x, x+8, ... and sweeps all nn column tiles of one row
// block before the next, so each X row block is read from HBM once and W
// stays in that XCD's L2.
template <int NJ, class Epi>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W,
                                                           int64_t M, int N, int K, int nm, int nn,
                                                           Epi epi) {
  constexpr int BM = 64 * NJ;      // block rows; each wave owns BM/2 rows x 64 columns
  // one LDS block: the three ring stages during the K loop (they reach the
  // loop as distinct restrict-qualified pointers), the output tile after it
  constexpr int kRing = 3 * (BM + kGN) * kRowB;
  constexpr int kTile = BM * kOutRowB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing > kTile ? kRing : kTile];
  __shared__ __attribute__((aligned(16))) float sbias[kGN];   // bias of the tile's columns (0 past N)
  uint8_t* const sX0 = smem;
  uint8_t* const sX1 = smem + BM * kRowB;
  uint8_t* const sX2 = smem + 2 * BM * kRowB;
  uint8_t* const sW0 = smem + 3 * BM * kRowB;
  uint8_t* const sW1 = sW0 + kGN * kRowB;
  uint8_t* const sW2 = sW0 + 2 * kGN * kRowB;

  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int slot = id >> 3;
  const int mb = (slot / nn) * 8 + xcd;
  const int nb = slot - (slot / nn) * nn;
  if (mb >= nm) return;
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
    xsrc[i] = X + gm * K + 8 * (lp ^ ((r >> 2) & 3));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (wave + 4 * i) + lr;
    const int gn = min(n0 + r, N - 1);
    wsrc[i] = W + static_cast<int64_t>(gn) * K + 8 * (lp ^ ((r >> 2) & 3));
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

  // Output tile through LDS. C^T accumulator: lane -> row j*32 + lane%32,
  // columns i*32 + 8*(r/4) + 4*h + r%4 of the wave's block.
  lds_barrier();   // every wave is done reading the ring
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ml = wm * 32 * NJ + j * 32 + l32;
    const int64_t m = m0 + ml;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * 64 + i * 32 + 8 * g + 4 * h;
        const float v[4] = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                            acc[i][j][4 * g + 3]};
        const float4 b = *reinterpret_cast<const float4*>(&sbias[nl]);
        const uint2 o = (m < M && n0 + nl < N) ? epi.pack(m, n0 + nl, v, b) : make_uint2(0, 0);
        *reinterpret_cast<uint2*>(smem + ml * kOutRowB + nl * 2) = o;
      }
  }
  lds_barrier();
  // 16 threads per 256-byte row segment, 16 rows per pass
#pragma unroll
  for (int it = 0; it < BM / 16; ++it) {
    const int row = it * 16 + (tid >> 4);
    const int nl = (tid & 15) * 8;
    const int64_t m = m0 + row;
    if (m < M && n0 + nl < N)
      epi.store8(m, n0 + nl, *reinterpret_cast<const uint4*>(smem + row * kOutRowB + nl * 2));
  }
}

// ---------------------------------------------------------------------------
// fp32: 16 x 16 output tile per block, K staged through LDS in steps of 16.
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
// 256-row ones would leave the 256 compute units with under two rounds of
// work.
template <class Epi>
hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int N, int K, Epi epi,
                            hipStream_t s) {
  const int nn = (N + kGN - 1) / kGN;
  const int64_t blocks256 = (M + 255) / 256 * nn;
  if (blocks256 >= 2 * 512) {
    const int nm = static_cast<int>((M + 255) / 256);
    const int grid = 8 * ((nm + 7) / 8) * nn;
    hipLaunchKernelGGL((gemm_bf16_kernel<4, Epi>), dim3(grid), dim3(256), 0, s, x, w, M, N, K, nm, nn, epi);
  } else {
    const int nm = static_cast<int>((M + 127) / 128);
    const int grid = 8 * ((nm + 7) / 8) * nn;
    hipLaunchKernelGGL((gemm_bf16_kernel<2, Epi>), dim3(grid), dim3(256), 0, s, x, w, M, N, K, nm, nn, epi);
  }
  return hipGetLastError();
}

hipError_t launch_proj_bf16(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  ProjEpi epi{a.bias,
              {static_cast<uint16_t*>(a.out[0]), static_cast<uint16_t*>(a.out[1]),
               static_cast<uint16_t*>(a.out[2]), static_cast<uint16_t*>(a.out[3])},
              a.K};
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
  OutEpiF32 epi{a.bias, static_cast<const float*>(a.x), static_cast<float*>(a.y), a.K};
  dim3 grid(static_cast<unsigned>((a.M + 15) / 16), (a.K + 15) / 16);
  hipLaunchKernelGGL(gemm_f32_kernel<OutEpiF32>, grid, dim3(256), 0, s,
                     static_cast<const float*>(a.g), static_cast<const float*>(a.w), a.M, a.K,
                     a.K, epi);
  return hipGetLastError();
}

}  // namespace hstu
