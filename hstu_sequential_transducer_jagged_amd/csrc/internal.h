// Internal declarations shared by the host ABI (api.cpp) and the HIP kernel
// translation units. Launchers enqueue on the given stream and return the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// Arguments of the jagged attention kernels (all pointers device memory).
struct AttnArgs {
  const void* q;             // [T, d] own queries
  const void* k;             // [T, d] own keys
  const void* v;             // [T, d] own values
  const void* ck;            // [Tc, d] cached keys or null
  const void* cv;            // [Tc, d] cached values or null
  const int64_t* offsets;    // [B+1]
  const int64_t* ts;         // [T]
  const int32_t* num_targets;// [B] or null
  const int64_t* c_offsets;  // [B+1] or null
  const int64_t* c_ts;       // [Tc] or null
  const float* pos_bias;     // [pos_len]
  const float* time_bias;    // [ntypes^2 * nb]: one table per (query type, key type) pair
  const int32_t* types;      // [T] token types (ntypes > 1) or null
  const int32_t* c_types;    // [Tc] cached token types (ntypes > 1) or null
  int ntypes;                // 1: untyped rab
  int linear;                // 1: parameter-free bias -m_p dp - m_t bucket, no tables
  float m_p, m_t;
  float* av;                 // [T, d] fp32 out
  int d_model;
  int num_heads;
  int head_dim;
  int pos_len;
  int pos_center;            // n_max - 1
  int nb;
  float alpha;
  int num_seqs;
  int max_seq_len;
  int max_cache_len;
  int no_self;               // targets do not see themselves
  int in_bf16;               // per-row kernel: q/k/v/ck/cv are bf16 (else fp32)
  int64_t total_tokens;      // T
  int* sched;                // bf16 path: work list built by the scheduling pass
  int sched_ready;           // bf16 path: the work list is already built (by the f1 launch)
  int bm;                    // bf16 path: queries per work item (64)
  int splits;                // bf16 path: key-range chunks per (sequence, query tile)
  float* partial;            // [splits, T, d] fp32 partial outputs when splits > 1
  // bf16 path, one head group covering d_model and splits == 1 only: when
  // fuse_ng is set the kernel writes G = (LayerNorm(AV) * gamma + beta) (.) U
  // to ng_g instead of AV (ng_g may alias ng_u)
  int fuse_ng;
  const void* ng_u;
  void* ng_g;
  const float* ng_gamma;
  const float* ng_beta;
  float ng_eps;
};

// Work decomposition of the bf16 attention (shared by the host plan and the
// kernels): queries per work item; the work list's header (one counter per
// XCD, then the total) ahead of the item ids; below kAttnSplitMinUnits items
// the key range of each item is split into up to kAttnMaxSplits chunks.
constexpr int kAttnBM = 64;
constexpr int kAttnBN = 32;   // keys per step of the bf16 kernel
constexpr int kAttnSchedHead = 9;
constexpr int64_t kAttnSplitMinUnits = 512;
constexpr int kAttnMaxSplits = 8;
// Heads per workgroup: the largest of 8, 4, 2, 1 dividing the head count.
int attn_heads_per_group(int num_heads);

// Launch plan of the bf16 attention for a batch shape: queries per work
// item, heads per workgroup, key-range chunks per item (1 unless the batch has
// too few items to fill the chip), and the workspace layout (the work list,
// then with splits > 1 the fp32 partial outputs).
struct AttnPlan {
  int bm;
  int heads_per_group;
  int splits;
  size_t sched_bytes;
  size_t workspace_bytes;
};
// max_splits caps the key-range splits (the allocation-free entry point
// lowers it until its workspace fits the static scratch).
AttnPlan attn_plan(int num_seqs, int max_seq_len, int num_heads, int64_t total_tokens, int d_model,
                   int max_splits = 8);
// Bytes of the static device scratch behind hstu_attn_fwd_noalloc, and its
// device address on the current device (resolved once per device).
constexpr size_t kAttnStaticScratchBytes = size_t{32} << 20;
hipError_t attn_static_scratch(void** ptr);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// Whether launch_attn_bf16 can fuse norm_gate for this shape (one head group
// per row, no key-range splits).
bool attn_can_fuse_norm_gate(int num_seqs, int max_seq_len, int num_heads, int64_t total_tokens,
                             int d_model);
// Per-row attention (one thread per query row), every option; fp32 inputs,
// or bf16 ones with head_dim 32 when a.in_bf16 is set.
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// C[M, N] = A[M, K] B[N, K]^T (+ epilogue). Both operands row-major with K
// contiguous (nn.Linear weight layout for B).
struct ProjArgs {
  const void* x;   // [M, K]
  const void* w;   // [N, K] (N = 4K)
  const float* bias;  // [N] or null
  void* out[4];    // U, V, Q, K  [M, K] each
  int64_t M;
  int K;           // d_model
  // bf16: when set, the launch also builds this attention's work list (one
  // extra workgroup), which the attention then takes as ready
  const AttnArgs* sched = nullptr;
};
struct OutArgs {
  const void* g;   // [M, K]
  const void* w;   // [K, K]
  const float* bias;  // [K] or null
  const void* x;   // [M, K] residual
  void* y;         // [M, K]
  int64_t M;
  int K;
};

// fp32 GEMM on the matrix cores: C[m, n] = sum_k A[m sam + k sak] B[k sbk + n sbn].
// epi 0: C = acc + bias[n] + addend[m, n] (each optional; addend row stride ldc);
// epi 1: C += acc atomically, K split over `splits` chunks (C zeroed by the caller);
// epi 2: outs[n / split][m * split + n % split] = SiLU(acc + bias[n]), and
//        C[m, n] = acc + bias[n] when C is set (split % 16 == 0, N <= 4 split).
// Returns hipErrorNotSupported, launching nothing, for operand layouts it does
// not take (each operand needs its k index or its m / n index contiguous,
// the other stride a multiple of 4, 16-byte aligned bases) and for products
// of fewer than 8 workgroups (128 x 128 tiles times K chunks).
struct GemmF32Args {
  const float* A;
  int64_t sam, sak;
  const float* B;
  int64_t sbk, sbn;
  float* C;
  int64_t ldc;
  const float* addend;
  const float* bias;
  float* outs[4];
  int split;
  int M, N;
  int64_t K, kchunk;
};
hipError_t launch_gemm_f32_mma(const GemmF32Args& a, int epi, int splits, hipStream_t s);

// bf16 products of the training layer: C[M, N] (fp32) = A[M, K] B[N, K]^T,
// A and B row-major bf16 with row strides lda, ldb (% 8 == 0) and K
// contiguous. K = splits * kc (kc % 32 == 0; rows zero-padded to that
// length). splits == 1: C + bias (+ addend, [M, ldc] fp32 or nullptr) is
// written to c (if not nullptr), and with act[0] set also SiLU of it split
// into the four [M, act_w] arrays act[0..3] (N == 4 act_w), and into bf16
// copies act16[i] where those are set; splits > 1 (no
// bias, addend or act): split s writes its partial product to
// c + s * M * ldc, and launch_sum_splits adds them up. N % 4 == 0,
// ldc % 4 == 0.
struct GemmBf16Args {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  float* c;
  int64_t ldc;
  const float* addend;
  int64_t M;
  int N;
  int kc;
  int splits;
  const float* bias = nullptr;
  float* act[4] = {nullptr, nullptr, nullptr, nullptr};
  int act_w = 0;
  uint16_t* act16[4] = {nullptr, nullptr, nullptr, nullptr};
};
hipError_t launch_gemm_bf16_f32(const GemmBf16Args& g, hipStream_t s);
// dst [rows, 3 cols] bf16 from src [rows, cols] fp32 (cols % 4 == 0): each
// value split as hi = bf16(x), lo = bf16(x - hi), the column blocks
// [hi | lo | hi] (lo_last 0) or [hi | hi | lo] (lo_last 1). A bf16 product of
// an lo_last-0 copy of A with an lo_last-1 copy of B, contracted over the
// 3 cols, is A B^T up to the lo*lo term (about 2^-16 relative per product).
hipError_t launch_to_bf16x3(const float* src, int64_t rows, int cols, uint16_t* dst, int lo_last, hipStream_t s);
// out[i] = sum over s < splits of part[s * n + i] (n % 4 == 0)
hipError_t launch_sum_splits(const float* part, int splits, int64_t n, float* out, hipStream_t s);
// dst[c * ld_dst + r] = bf16(src[r * ld_src + c]) for r < rows, c < cols, and
// 0 for rows <= r < ld_dst: the transposed bf16 copy, zero-padded along r
// (cols % 4 == 0, ld_src % 4 == 0, ld_dst % 8 == 0). With dst_rows, also
// dst_rows[r * ld_rows + c] = bf16(src[r * ld_src + c]) for r < rows, c < cols
// (ld_rows % 4 == 0, 8-byte aligned); with rows_x3, the rows of
// launch_to_bf16x3(lo_last = 0) instead (ld_rows >= 3 cols). With colsum,
// colsum[c] += sum over r of src[r * ld_src + c] (atomic fp32 adds).
hipError_t launch_to_bf16_t(const float* src, int64_t ld_src, int64_t rows, int cols, uint16_t* dst,
                            int64_t ld_dst, hipStream_t s, uint16_t* dst_rows = nullptr, int64_t ld_rows = 0,
                            bool rows_x3 = false, float* colsum = nullptr);
// The same transposed copy from a bf16 source (exact).
hipError_t launch_bf16_t(const uint16_t* src, int64_t ld_src, int64_t rows, int cols, uint16_t* dst,
                         int64_t ld_dst, hipStream_t s);
hipError_t launch_proj_bf16(const ProjArgs& a, hipStream_t s);
hipError_t launch_proj_f32(const ProjArgs& a, hipStream_t s);
hipError_t launch_out_bf16(const OutArgs& a, hipStream_t s);
hipError_t launch_out_f32(const OutArgs& a, hipStream_t s);

struct NormGateArgs {
  const float* av;   // [M, d]
  const void* u;     // [M, d]
  const float* gamma;
  const float* beta;
  void* g;           // [M, d]
  int64_t M;
  int d;
  float eps;
};
hipError_t launch_norm_gate_bf16(const NormGateArgs& a, hipStream_t s);
hipError_t launch_norm_gate_f32(const NormGateArgs& a, hipStream_t s);

// Y = LayerNorm_d(X) * gamma + beta, row by row (the optional input norm).
struct LayerNormArgs {
  const void* x;     // [M, d] dtype
  const float* gamma;
  const float* beta;
  void* y;           // [M, d] dtype
  int64_t M;
  int d;
  float eps;
};
hipError_t launch_layernorm_bf16(const LayerNormArgs& a, hipStream_t s);
hipError_t launch_layernorm_f32(const LayerNormArgs& a, hipStream_t s);

// ---- backward (fp32, plain causal attention) ----
struct BwdAttnArgs {
  const float* q;            // [T, d] (row stride d)
  const float* k;
  const float* v;
  const float* dav;          // [T, d] gradient of AV
  // bf16 copies of q, k, v, dav (the bf16 backward reads these instead)
  const uint16_t* q16;
  const uint16_t* k16;
  const uint16_t* v16;
  const uint16_t* dav16;
  const int64_t* offsets;    // [B+1]
  const int64_t* ts;         // [T]
  const float* pos_bias;
  const float* time_bias;
  float* dq;                 // [T, ld_dz] blocks of dZ
  float* dk;
  float* dv;
  float* dpos;               // [pos_len], accumulated
  float* dtime;              // [nb], accumulated
  float* av;                 // [T, d] forward output (launch_attn_train_fwd)
  int ld_dz;
  int d_model, num_heads, head_dim, pos_len, pos_center, nb;
  float alpha;
  int num_seqs, max_seq_len;
};
// fp32 attention on the matrix cores, plain causal (no targets, no cache),
// head_dim 32 or 64: the forward AV, and the backward (dQ, dK, dV, table
// gradients accumulated into dpos/dtime).
bool attn_train_supported(int head_dim);
hipError_t launch_attn_train_fwd(const BwdAttnArgs& a, hipStream_t s);
hipError_t launch_attn_bwd_f32(const BwdAttnArgs& a, hipStream_t s);
// The same backward on the bf16 matrix cores, from a.q16/k16/v16/dav16
// (head_dim 32 or 64); the outputs and table gradients as above.
hipError_t launch_attn_bwd_bf16(const BwdAttnArgs& a, hipStream_t s);
// Plain causal AV (fp32, row stride d_model) from a.q16/k16/v16 on the bf16
// matrix cores, head_dim 32 or 64: the bf16 forward for head dimensions the
// tiled bf16 kernel does not take.
hipError_t launch_attn_fwd_bf16_rows(const BwdAttnArgs& a, hipStream_t s);
// dst[i] = bf16(src[i]) (round to nearest even), n a multiple of 4.
hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
// C[m, n] = sum_k A[m sam + k sak] B[k sbk + n sbn] (+ bias[n] + addend[m, n]);
// splits > 1: K split over blocks whose sums are added atomically into C
// (zeroed beforehand, no bias or addend).
hipError_t launch_gemm_f32s(const float* A, int64_t sam, int64_t sak, const float* B, int64_t sbk,
                            int64_t sbn, float* C, int64_t ldc, const float* addend, const float* bias,
                            int M, int N, int64_t K, int splits, hipStream_t s);
// Zeroes up to kZeroListMax buffers (p[i], n[i] floats) in one launch.
constexpr int kZeroListMax = 10;
struct ZeroList {
  float* p[kZeroListMax];
  int64_t n[kZeroListMax];
  int count;
};
hipError_t launch_fill_zero_list(const ZeroList& z, hipStream_t s);
// Input LayerNorm backward (d <= 1024): dx = dy + LN'(x)^T dxn, with the
// statistics recomputed from x; dgamma/dbeta += column sums of dxn * xhat
// and dxn.
hipError_t launch_ln1_bwd(const float* x, const float* dxn, const float* dy, const float* gamma, float* dx,
                          float* dgamma, float* dbeta, int64_t M, int d, float eps, hipStream_t s);
hipError_t launch_colsum(const float* X, int64_t ldx, int64_t M, int N, float* out, hipStream_t s);
hipError_t launch_ln_gate_fwd(const float* av, const float* u, const float* gamma, const float* beta,
                              float* nhat, float* rstd, float* g, uint16_t* g16, int64_t M, int d, float eps,
                              hipStream_t s);
hipError_t launch_ln_gate_bwd(const float* dg, const float* u, const float* nhat, const float* rstd,
                              const float* gamma, const float* beta, float* du, int64_t ldu, float* dav,
                              uint16_t* dav16, float* dgamma, float* dbeta, int64_t M, int d, hipStream_t s);
hipError_t launch_silu_bwd(float* dz, const float* z, int64_t n, hipStream_t s);
// dZ = dz . SiLU'(z) over [T, n] fp32 (not written back): dz16 [T, n] bf16,
// dzt [n, tp] bf16 (dZ^T, zero for T <= t < tp), and db1[c] += sum_t dZ[t, c]
// (n % 4 == 0, tp % 8 == 0, tp >= T).
hipError_t launch_silu_bwd_bf16(const float* dz, const float* z, int64_t T, int n, uint16_t* dz16,
                                uint16_t* dzt, int64_t tp, float* db1, hipStream_t s);

// Error channel of the C ABI (hstu_last_error), for entry points defined
// outside api.cpp: api_fail records a message and returns code.
int api_fail(int code, const char* fmt, ...);
void api_ok();

// dst[r] = src[rows[r]] for r < n, row_bytes per row (a multiple of 8);
// rows are clamped to [0, src_rows).
hipError_t launch_gather_rows(int64_t n, int row_bytes, const int64_t* rows, int64_t src_rows,
                              const void* src, void* dst, hipStream_t s);

// Per-sequence concatenation of two K/V caches: rows of sequence b in out
// are [a's rows of b, then n's rows of b]; out offsets = a + n offsets.
struct CacheConcatArgs {
  const int64_t* a_off;  // [B+1]
  const int64_t* a_ts;
  const void* a_k;
  const void* a_v;
  const int64_t* n_off;  // [B+1]
  const int64_t* n_ts;
  const void* n_k;
  const void* n_v;
  int64_t* out_off;      // [B+1]
  int64_t* out_ts;
  void* out_k;
  void* out_v;
  int64_t rows;          // a_T + n_T
  int64_t a_T;           // rows of a and of n (source rows are clamped to them)
  int64_t n_T;
  int B;
  int row_bytes;         // d * element size, a multiple of 16
};
hipError_t launch_cache_concat(const CacheConcatArgs& a, hipStream_t s);

// pos[i] = -m_p * (i - (len - 1) / 2), time[p * nb + b] = -m_t * b for each
// of `pairs` type-pair tables: the tables that make the table bias equal the
// parameter-free position/time bias.
hipError_t launch_linear_bias_tables(float m_p, float m_t, int pos_len, int num_buckets, int pairs,
                                     float* pos, float* time, hipStream_t s);

struct EmbedArgs {
  const void* item;
  const void* action;
  const int64_t* ids;
  const int32_t* acts;
  void* x;
  int64_t T;
  int64_t num_items;
  int num_actions;
  int d;
};
hipError_t launch_embed_bf16(const EmbedArgs& a, hipStream_t s);
hipError_t launch_embed_f32(const EmbedArgs& a, hipStream_t s);

}  // namespace hstu
