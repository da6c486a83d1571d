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
  const float* time_bias;    // [nb]
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
  int64_t total_tokens;      // T
  int* sched;                // bf16 path: work list built by the scheduling pass
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

// bf16 attention: number of key-range chunks per work item (1 unless the
// batch has too few (sequence, query tile) items to fill the chip).
int attn_splits(int num_seqs, int max_seq_len);
// Workspace bytes of the bf16 attention: the work list, then (splits > 1) the
// partial outputs.
size_t attn_sched_bytes(int num_seqs, int max_seq_len);
size_t attn_workspace_bytes(int num_seqs, int max_seq_len, int64_t total_tokens, int d_model);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// Whether launch_attn_bf16 can fuse norm_gate for this shape (one head group
// per row, no key-range splits).
bool attn_can_fuse_norm_gate(int num_heads, int num_seqs, int max_seq_len);
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
// C[m, n] = sum_k A[m sam + k sak] B[k sbk + n sbn] (+ bias[n] + addend[m, n]);
// splits > 1: K split over blocks whose sums are added atomically into C
// (zeroed beforehand, no bias or addend).
hipError_t launch_gemm_f32s(const float* A, int64_t sam, int64_t sak, const float* B, int64_t sbk,
                            int64_t sbn, float* C, int64_t ldc, const float* addend, const float* bias,
                            int M, int N, int64_t K, int splits, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
// Input LayerNorm backward (d <= 1024): dx = dy + LN'(x)^T dxn, with the
// statistics recomputed from x; dgamma/dbeta += column sums of dxn * xhat
// and dxn.
hipError_t launch_ln1_bwd(const float* x, const float* dxn, const float* dy, const float* gamma, float* dx,
                          float* dgamma, float* dbeta, int64_t M, int d, float eps, hipStream_t s);
hipError_t launch_colsum(const float* X, int64_t ldx, int64_t M, int N, float* out, hipStream_t s);
hipError_t launch_ln_gate_fwd(const float* av, const float* u, const float* gamma, const float* beta,
                              float* nhat, float* rstd, float* g, int64_t M, int d, float eps,
                              hipStream_t s);
hipError_t launch_ln_gate_bwd(const float* dg, const float* u, const float* nhat, const float* rstd,
                              const float* gamma, const float* beta, float* du, int64_t ldu, float* dav,
                              float* dgamma, float* dbeta, int64_t M, int d, hipStream_t s);
hipError_t launch_silu_bwd(float* dz, const float* z, int64_t n, hipStream_t s);

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

// pos[i] = -m_p * (i - (len - 1) / 2), time[b] = -m_t * b: the tables that
// make the table bias equal the parameter-free position/time bias.
hipError_t launch_linear_bias_tables(float m_p, float m_t, int pos_len, int num_buckets,
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
