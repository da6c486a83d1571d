/*
 * hstu.h — C ABI of the MI355X (gfx950) HSTU jagged layer forward.
 *
 * One HSTU layer on jagged (offset-packed, variable-length) sequences:
 *
 *   U, V, Q, K = Split(SiLU(X W1^T + b1))                       (projection)
 *   AV_h       = (SiLU(alpha Q_h K_h^T + rab_{p,t}) * Mask) V_h  (per head)
 *   Y          = X + (LayerNorm(AV) * gamma + beta) (.) U  W2^T + b2
 *
 * The three equations are the ones of "万亿参数推荐大模型：HSTU 架构如何超越
 * 传统 Self-Attention" §2.1 (and of "从自注意力到 HSTU：解构下一代推荐系统引擎"
 * part 2, steps 1-3); the residual is that page's block-diagram skip
 * connection. There is no softmax and no normalisation of the SiLU weights
 * ("HSTU：Scaling Law 的首次探索" §7.1.4, innovation 1).
 *
 * rab_{p,t}(i, j) = pos_bias[(p_i - p_j) + n_max - 1]
 *                 + time_bias[min(nb - 1, floor(log2(|t_i - t_j| + 1)))]
 * is shared by all heads; position and real-time differences follow
 * §7.1.4 innovation 2 of the chapter-7.1 page, the bucketed time difference
 * eq. 6.2.6 of "6.2. HSTU的工程突破". The floor(log2) is exact (integer).
 * Two options of the same term (hstu_layer_desc): token types, where the
 * time table is one table per ordered (query type, key type) pair, the
 * type-aware bias of §7.1.4 innovation 2; and the parameter-free bias of
 * eq. 6.2.6, -m_p (p_i - p_j) - m_t bucket, computed in the kernels.
 *
 * Visibility. Within sequence b the keys are [the cache rows of b, then the
 * call's own tokens of b]. Key j is visible to query i iff j is a cache row,
 * or j <= i and (j is not a target or j == i) (own-token indices; the last
 * num_targets[b] own tokens are targets). Plain causal attention is the case
 * without cache and targets. Targets and the cache implement candidate
 * scoring with micro-batches over a cached history (M-FALCON, §7.1.5 of the
 * chapter-7.1 page; the candidate mask of Fig. 6.2.2 of the GenRank page).
 *
 * Positions. Cache rows of b: 0 .. n_b-1 (n_b = its cache length). Own
 * non-targets: n_b + j. All targets of b share n_b + (L_b - m_b).
 *
 * Conventions for every entry point:
 *  - returns an hstu_status; on error nothing has been enqueued (argument
 *    errors) or the outputs are undefined (HSTU_E_DEVICE); a message is
 *    available from hstu_last_error() on the calling thread;
 *  - asynchronous: work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and the call returns without waiting;
 *  - never allocates device memory; the caller owns every buffer;
 *  - "device" pointers are HIP device memory; all arrays are dense and
 *    row-major; activations [T, d_model] must be 16-byte aligned;
 *  - outputs must not alias inputs;
 *  - device-resident index data (offsets, num_targets, timestamps) are not
 *    validated by the fast path; hstu_check_inputs() validates them.
 *
 * dtype HSTU_BF16: X, W1, W2, U/V/Q/K, G, Y, cache K/V are bf16 (raw 16-bit
 * patterns), arithmetic accumulates in fp32. HSTU_F32: all of those fp32.
 * Bias tables, linear biases, LayerNorm parameters and AV are always fp32.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 11

typedef enum {
  HSTU_OK = 0,
  HSTU_E_INVAL = -1,        /* bad argument (null pointer, size, alignment, range) */
  HSTU_E_UNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim) */
  HSTU_E_WORKSPACE = -3,    /* workspace too small */
  HSTU_E_DEVICE = -4,       /* HIP runtime error (launch, device query, copy) */
  HSTU_E_DATA = -5          /* hstu_check_inputs found inconsistent device data */
} hstu_status;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype;

/* Source of rab (hstu_layer_desc.bias_mode). */
typedef enum { HSTU_BIAS_TABLES = 0, HSTU_BIAS_LINEAR = 1 } hstu_bias_mode;

#define HSTU_MAX_TOKEN_TYPES 4

/* Host-side layer description, passed by pointer, read during the call only. */
typedef struct {
  int32_t d_model;          /* == num_heads * head_dim */
  int32_t num_heads;
  int32_t head_dim;         /* 32 or 64 (bf16 head_dim 32: see hstu_attn_fwd) */
  int32_t dtype;            /* hstu_dtype */
  float alpha;              /* score scale, 1e-6 <= |alpha| <= 1e6 (1.0 by default) */
  float ln_eps;             /* LayerNorm epsilon, >= 0 (1e-5 by default) */
  int32_t pos_table_len;    /* 2*n_max - 1 (odd); index = (p_i - p_j) + n_max - 1 */
  int32_t num_time_buckets; /* 1..64 (32 by default) */
  int32_t input_norm;       /* 0 (default) or 1: hstu_layer_fwd first applies the input
                               LayerNorm (params ln1_gamma/ln1_beta, eps ln_eps) to X,
                               the Norm1 of the block diagram of "万亿参数推荐大模型…"
                               §2.1; the residual still adds the raw X */
  int32_t target_no_self;   /* 0 (default) or 1: a target then sees the cache and the
                               non-targets only, not itself (the literal reading of the
                               M-FALCON mask of "HSTU：Scaling Law 的首次探索" §7.1.5:
                               a candidate attends to the user history) */
  int32_t num_token_types;  /* 0 or 1 (default): untyped rab. 2..HSTU_MAX_TOKEN_TYPES: the
                               type-aware rab of "HSTU：Scaling Law 的首次探索" §7.1.4
                               innovation 2 (content and action tokens decay differently):
                               time_bias then holds num_token_types^2 tables of
                               num_time_buckets entries, the pair (query type a, key type b)
                               at offset (a * num_token_types + b) * num_time_buckets; the
                               position table stays shared. Token types come from
                               hstu_jagged.token_types (and the cache's); forward only */
  int32_t bias_mode;        /* hstu_bias_mode. HSTU_BIAS_LINEAR: rab(i, j) = -linear_m_p
                               (p_i - p_j) - linear_m_t bucket(t_i - t_j), the parameter-free
                               bias of "6.2. HSTU的工程突破" eq. 6.2.6 (slopes shared by all
                               heads), computed by the kernels with no tables: pos_bias and
                               time_bias are not read (may be NULL). Untyped, forward only */
  float linear_m_p;         /* slopes of HSTU_BIAS_LINEAR, finite */
  float linear_m_t;
  int32_t attn_bwd_bf16;    /* 0 (default) or 1, read by the training entry points
                               (hstu_layer_bwd, hstu_layer_fwd_train,
                               hstu_layer_bwd_after_fwd): the attention backward runs on
                               the bf16 matrix cores, and so does the attention forward
                               of the training layer (the recompute, and
                               hstu_layer_fwd_train's), on the forward path's kernels
                               with fp32 AV. Q, K, V and dAV are rounded to bf16 once, P and dS
                               as the operands of their products; every sum is fp32. Other
                               steps stay fp32 (see gemm_bwd_bf16 for the products).
                               Gradients then agree with the fp32 ones to the bf16
                               tolerance: matrices per row to 2e-2, vector entries to 2e-2
                               of themselves or 2^-7 of the magnitude of the terms they
                               sum */
  int32_t gemm_bwd_bf16;    /* 0 (default) or 1, read by the training entry points: every
                               product of the training layer runs on the bf16 matrix cores:
                               f1 (Z = Xin W1^T + b1 with the SiLU split, Xin the input of
                               f1), f2 of hstu_layer_fwd_train, and the backward's
                               dG = dY W2, dW2 = dY^T G, dW1 = dZ^T Xin and dX = dZ W1.
                               Their operands are rounded to bf16 once (f1's are split
                               into bf16 hi and lo parts, three products contracted
                               together, since f1 feeds every gradient), the sums and
                               outputs are fp32; the weight gradients sum over the tokens
                               in fixed splits (no atomics). Independent of
                               attn_bwd_bf16. Gradients then agree with the fp32 ones to
                               the bf16 tolerance: matrices per row to 2e-2, vector
                               entries to 2e-2 of themselves or 2^-7 of the magnitude of
                               the terms they sum. The workspace grows by the bf16
                               operand copies */
} hstu_layer_desc;

/* A jagged batch of the call's own tokens. */
typedef struct {
  int32_t num_seqs;             /* B >= 0 (host) */
  int32_t max_seq_len;          /* >= every L_b (host); sizes the launch grid */
  int64_t total_tokens;         /* T = offsets[B] (host) */
  const int64_t *offsets;       /* device [B+1]: offsets[0] = 0, nondecreasing, offsets[B] = T */
  const int64_t *timestamps;    /* device [T], int64 seconds (any order) */
  const int32_t *num_targets;   /* device [B] or NULL: the last m_b tokens of b are targets,
                                   0 <= m_b <= L_b */
  const int32_t *token_types;   /* device [T] with num_token_types > 1 (each in
                                   [0, num_token_types)), else unused (may be NULL) */
} hstu_jagged;

/* Optional cached history (keys/values visible to every own token of the
 * same sequence). Pass NULL when there is none. */
typedef struct {
  const int64_t *offsets;       /* device [B+1] rows of k/v per sequence (same B as the batch) */
  const int64_t *timestamps;    /* device [cache_T] */
  const void *k;                /* device [cache_T, d_model], dtype */
  const void *v;                /* device [cache_T, d_model], dtype */
  int32_t max_len;              /* >= every cache length (host) */
  int64_t total_tokens;         /* cache_T (host) */
  const int32_t *token_types;   /* device [cache_T] with num_token_types > 1, else unused */
} hstu_kv_cache;

/* Layer parameters: device pointers, caller-owned. */
typedef struct {
  const void *w1;               /* [4d, d] dtype, nn.Linear layout (out x in) */
  const float *b1;              /* [4d] or NULL (zeros) */
  const void *w2;               /* [d, d] dtype */
  const float *b2;              /* [d] or NULL (zeros) */
  const float *ln_gamma;        /* [d] or NULL (ones) */
  const float *ln_beta;         /* [d] or NULL (zeros) */
  const float *pos_bias;        /* [pos_table_len]; unused with HSTU_BIAS_LINEAR */
  const float *time_bias;       /* [num_time_buckets], or [T^2 * num_time_buckets] with
                                   T = num_token_types > 1; unused with HSTU_BIAS_LINEAR */
  const float *ln1_gamma;       /* [d] or NULL (ones): input LayerNorm, read if input_norm */
  const float *ln1_beta;        /* [d] or NULL (zeros) */
} hstu_layer_params;

/* Gradients of one layer (hstu_layer_bwd): device fp32 buffers, overwritten. */
typedef struct {
  float *dw1;     /* [4d, d] */
  float *db1;     /* [4d] */
  float *dw2;     /* [d, d] */
  float *db2;     /* [d] */
  float *dgamma;  /* [d] */
  float *dbeta;   /* [d] */
  float *dpos;    /* [pos_table_len] */
  float *dtime;   /* [num_time_buckets] */
  float *dln1_gamma; /* [d], with desc->input_norm (else unused, may be NULL) */
  float *dln1_beta;  /* [d], likewise */
} hstu_layer_grads;

/* ABI version of the loaded library (HSTU_ABI_VERSION). */
int hstu_abi_version(void);

/* Message describing the last error on this thread ("" if none). Valid until
 * the next call on the same thread. */
const char *hstu_last_error(void);

/* Pointwise projection, "万亿参数推荐大模型…" §2.1 first equation:
 *   [U | V | Q | K] = SiLU(x W1^T + b1), split into four [T, d] outputs in
 *   the order U, V, Q, K (head h owns columns [h*dh, (h+1)*dh) of each).
 * x [T, d], u/v/q/k [T, d] (dtype). T >= 0. */
int hstu_proj_fwd(const hstu_layer_desc *desc, const hstu_layer_params *params, int64_t T,
                  const void *x, void *u, void *v, void *q, void *k, void *stream);

/* Workspace bytes hstu_attn_fwd needs for this batch. bf16, head_dim 64: the work list
 * of its scheduling pass, 4 * (9 + U) bytes rounded up to 256, with
 * U = I * S units, I = num_seqs * ceil(max_seq_len / 64) (sequence, query
 * tile) items and S key-range splits per item (S = 1 when I >= 512, else
 * min(8, ceil(512 / I)); then, when S > 1, S partial outputs of
 * total_tokens x d_model fp32. f32, and bf16 with head_dim 32: 0. */
size_t hstu_attn_workspace_size(const hstu_layer_desc *desc, const hstu_jagged *jagged);

/* Spatial aggregation, §2.1 second equation, with the visibility, position
 * and bias rules above:
 *   av[i, h*dh:(h+1)*dh] = sum_{j visible} SiLU(alpha q_i.k_j + rab(i, j)) v_j
 * q, k, v [T, d] (dtype, own tokens of `jagged`); cache may be NULL;
 * pos_bias [pos_table_len], time_bias [num_time_buckets], or
 * [num_token_types^2 * num_time_buckets] with token types (fp32; neither is
 * read with HSTU_BIAS_LINEAR); token types outside [0, num_token_types) are
 * clamped by the kernels (hstu_check_inputs() reports them);
 * av [T, d] fp32 output. workspace: device, 256-byte aligned, at least
 * hstu_attn_workspace_size() bytes (may be NULL when that is 0); its
 * contents are scratch. Every visible position difference must lie in
 * the table: per sequence, C_b + L_b - 1 <= n_max - 1 without targets and
 * C_b + (L_b - m_b) <= n_max - 1 with m_b > 0 targets (C_b = cache length).
 * Without num_targets the call checks max_seq_len + cache max_len <= n_max
 * (HSTU_E_INVAL); with targets the bound depends on device data and only
 * hstu_check_inputs() checks it (the kernels clamp table indices, so a
 * violation never reads out of bounds). Lengths above max_seq_len are a
 * contract violation: their query tiles past max_seq_len are not computed.
 * bf16 with head_dim 32 runs plain causal batches on the bf16 matrix cores
 * (32-query blocks per head); with targets, a cache, token types or
 * HSTU_BIAS_LINEAR it runs on a per-row kernel with fp32 arithmetic, which
 * is correct at any size but not tuned for speed. */
int hstu_attn_fwd(const hstu_layer_desc *desc, const hstu_jagged *jagged,
                  const hstu_kv_cache *cache, const void *q, const void *k, const void *v,
                  const float *pos_bias, const float *time_bias, float *av, void *workspace,
                  size_t workspace_bytes, void *stream);

/* hstu_attn_fwd without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The work list and the partial outputs
 * live in a static device array of HSTU_ATTN_STATIC_SCRATCH_BYTES (32 MiB),
 * one per device, held until the process ends. Arguments and results are
 * those of hstu_attn_fwd; the key-range splits are capped so that they fit
 * the array, and where the cap applies the fp32 partial sums are added in a
 * different grouping (results agree to rounding; bitwise otherwise). A batch
 * whose work list alone exceeds the array returns HSTU_E_WORKSPACE. Every
 * call on a device shares that device's array, so calls that overlap on one
 * device race; every call overwrites all it reads, nothing needs clearing.
 * Allocates nothing. */
#define HSTU_ATTN_STATIC_SCRATCH_BYTES (32u << 20)
int hstu_attn_fwd_noalloc(const hstu_layer_desc *desc, const hstu_jagged *jagged,
                          const hstu_kv_cache *cache, const void *q, const void *k, const void *v,
                          const float *pos_bias, const float *time_bias, float *av, void *stream);

/* Pointwise transformation, first half (§2.1 third equation and the block
 * diagram: LayerNorm, then the product with U):
 *   g = (LayerNorm_d(av) * gamma + beta) (.) u
 * LayerNorm over all d features with the biased variance and desc->ln_eps.
 * av [T, d] fp32, u and g [T, d] dtype (g may equal u: in place). */
int hstu_norm_gate_fwd(const hstu_layer_desc *desc, int64_t T, const float *av, const void *u,
                       const float *gamma, const float *beta, void *g, void *stream);

/* Input LayerNorm, the Norm1 that the block diagram of "万亿参数推荐大模型…"
 * §2.1 draws before f1 (the layer equations have none; hstu_layer_fwd
 * applies it when desc->input_norm is 1):
 *   y = LayerNorm_d(x) * gamma + beta
 * over all d features with the biased variance and desc->ln_eps. x, y
 * [T, d] dtype (y must not alias x); gamma/beta [d] fp32 or NULL. */
int hstu_layernorm_fwd(const hstu_layer_desc *desc, int64_t T, const void *x, const float *gamma,
                       const float *beta, void *y, void *stream);

/* Tables of the parameter-free relative bias of "6.2. HSTU的工程突破"
 * eq. 6.2.6 (ALiBi's eq. 6.2.5 extended to time), with scalar slopes shared
 * by all heads:
 *   pos_bias[i]  = -m_p * (i - (n_max - 1))     i < pos_table_len
 *   time_bias[b] = -m_t * b                     b < num_time_buckets
 * With them, the table bias of every entry point equals
 * -m_p (p_i - p_j) - m_t bucket(t_i - t_j) exactly up to one fp32 rounding
 * of each product. pos_bias [pos_table_len], time_bias [num_time_buckets]
 * (with num_token_types > 1, every one of the T^2 pair tables gets the same
 * values): device fp32 outputs, overwritten. m_p, m_t finite.
 * desc->bias_mode = HSTU_BIAS_LINEAR computes the same bias inside the
 * attention kernels instead, with no tables. */
int hstu_linear_bias_tables(const hstu_layer_desc *desc, float m_p, float m_t, float *pos_bias,
                            float *time_bias, void *stream);

/* Per-sequence concatenation of two K/V caches, for candidate scoring across
 * requests (M-FALCON, "HSTU：Scaling Law 的首次探索" §7.1.5: a user's later
 * request reuses the cached history and adds the tokens that arrived since
 * it was cached):
 *   rows of sequence b in out = [a's rows of b, then n's rows of b]
 *   out_offsets[b] = a->offsets[b] + n->offsets[b]        (b = 0..num_seqs)
 * a and n: num_seqs sequences each (offsets [num_seqs+1], timestamps, k, v
 * [total_tokens, d] dtype; max_len unused). Typically a is the cache of the
 * earlier request and n the K/V (hstu_layer_fwd k_out/v_out) of the new
 * tokens, computed with a as their cache. Outputs: out_offsets
 * [num_seqs+1], out_timestamps [a_T + n_T] int64, out_k/out_v
 * [a_T + n_T, d] dtype; none may alias an input. Rows are read within
 * each input's total_tokens even if its device offsets are inconsistent. */
int hstu_kv_cache_concat(const hstu_layer_desc *desc, int32_t num_seqs, const hstu_kv_cache *a,
                         const hstu_kv_cache *n, int64_t *out_offsets, int64_t *out_timestamps,
                         void *out_k, void *out_v, void *stream);

/* Stochastic Length, "HSTU：Scaling Law 的首次探索" §7.1.5 (the page prints
 * N_{alpha/2} and N_alpha; read as powers), on the HOST (a data-loader step):
 * a sequence of length n > N^(alpha/2), N = n_max, is with probability
 *   p = 1 - N^alpha / n^2        (truncated iff u[b] < p, fp64)
 * replaced by k = floor(N^(alpha/2)) of its tokens: those with the smallest
 * keys (ties to the earlier token), kept in their original order. The page
 * does not say how the subsequence is sampled; this is the reading taken.
 * Otherwise the sequence is kept whole; alpha = 2 never truncates.
 * Host arrays: offsets [num_seqs+1] (start at 0, nondecreasing), u
 * [num_seqs] in [0, 1], keys [T] finite (T = offsets[num_seqs]); outputs
 * out_offsets [num_seqs+1] and rows (capacity rows_capacity >= T): the
 * source row of every kept token, sequence-major; *out_total = kept rows.
 * alpha in (0, 2], n_max >= 1. Deterministic for given inputs. */
int hstu_stochastic_length(int32_t num_seqs, const int64_t *offsets, double alpha, int64_t n_max,
                           const double *u, const double *keys, int64_t *out_offsets,
                           int64_t *rows, int64_t rows_capacity, int64_t *out_total);

/* Row gather (to build the sampled batch on the device):
 *   dst[r] = src[rows[r]]   r < n, row_bytes bytes per row
 * rows: device int64 [n], clamped to [0, src_rows); src, dst: device,
 * 8-byte aligned, row_bytes a positive multiple of 8; dst must not alias
 * src. */
int hstu_gather_rows(int64_t n, int32_t row_bytes, const int64_t *rows, int64_t src_rows,
                     const void *src, void *dst, void *stream);

/* Pointwise transformation, second half: y = x + g W2^T + b2
 * (f2 with the residual connection). g, x, y [T, d] dtype. */
int hstu_out_fwd(const hstu_layer_desc *desc, int64_t T, const void *g, const void *x,
                 const void *w2, const float *b2, void *y, void *stream);

/* Workspace bytes hstu_layer_fwd needs for this batch (host fields of
 * `jagged` only; one more [T, d] dtype buffer when desc->input_norm). */
size_t hstu_layer_workspace_size(const hstu_layer_desc *desc, const hstu_jagged *jagged);

/* One full layer: [input LayerNorm ->] projection -> attention -> norm/gate
 * -> f2 + residual (the residual adds the raw x).
 * x, y [T, d] dtype (y must not alias x). k_out / v_out: NULL, or [T, d]
 * dtype buffers that receive this call's K and V (to build a cache for later
 * calls). workspace: device, >= hstu_layer_workspace_size() bytes, 256-byte
 * aligned. */
int hstu_layer_fwd(const hstu_layer_desc *desc, const hstu_layer_params *params,
                   const hstu_jagged *jagged, const hstu_kv_cache *cache, const void *x,
                   void *y, void *k_out, void *v_out, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Workspace bytes of hstu_layer_bwd: 17 [T, d] fp32 buffers (18 with
 * desc->input_norm) plus T floats (each rounded up to 256 bytes). */
size_t hstu_layer_bwd_workspace_size(const hstu_layer_desc *desc, const hstu_jagged *jagged);

/* Backward pass of one layer for generative training ("HSTU：Scaling Law 的
 * 首次探索" §7.1.5: a causal forward over whole sequences), through the three
 * equations of "万亿参数推荐大模型…" §2.1 and the residual: given dy =
 * dL/dY, writes dx = dL/dX and every parameter gradient, including those of
 * the position and time tables (each visible pair adds its score gradient,
 * summed over heads, to the entries it read). Recomputes the forward.
 * With desc->input_norm the gradient also runs through the input LayerNorm
 * (params ln1_gamma/ln1_beta, NULL meaning ones/zeros) into dx, and
 * grads->dln1_gamma/dln1_beta must be set.
 * Supported: dtype HSTU_F32, plain causal attention (jagged->num_targets
 * NULL, no cache), the untyped table bias (num_token_types <= 1,
 * HSTU_BIAS_TABLES), total_tokens and max_seq_len * d_model below 2^31,
 * d_model <= 1024; else HSTU_E_UNSUPPORTED.
 * x, dy, dx [T, d] fp32 (dx must not alias x or dy); grads: all eight
 * pointers non-NULL. workspace: device, 256-byte aligned, >=
 * hstu_layer_bwd_workspace_size(). Gradient sums use fp32 atomics, so
 * their last bits may vary from run to run. */
int hstu_layer_bwd(const hstu_layer_desc *desc, const hstu_layer_params *params,
                   const hstu_jagged *jagged, const void *x, const void *dy, void *dx,
                   const hstu_layer_grads *grads, void *workspace, size_t workspace_bytes,
                   void *stream);

/* A training step in two calls, without the backward's forward recompute.
 * hstu_layer_fwd_train: the layer forward in fp32 (same equations and
 * support as hstu_layer_bwd: HSTU_F32, plain causal attention; the attention
 * on bf16 with desc->attn_bwd_bf16), writing y [T, d] (must not alias x) and keeping in `workspace`
 * (hstu_layer_bwd_workspace_size() bytes, 256-byte aligned) the activations
 * the backward reads: Z, U, V, Q, K, AV, the normalised AV, 1/sigma and G
 * (and LayerNorm(X) with input_norm; with the bf16 flags also bf16 copies of
 * Q, K, V and, with gemm_bwd_bf16, of the f1 input transposed, G being kept
 * in bf16 only).
 * hstu_layer_bwd_after_fwd: the backward of hstu_layer_bwd, reading those
 * activations instead of recomputing them; desc, params, jagged, x and the
 * workspace must be those of the hstu_layer_fwd_train call, with the
 * workspace untouched in between (it is not checked). Same errors as
 * hstu_layer_bwd. */
int hstu_layer_fwd_train(const hstu_layer_desc *desc, const hstu_layer_params *params,
                         const hstu_jagged *jagged, const void *x, void *y, void *workspace,
                         size_t workspace_bytes, void *stream);
int hstu_layer_bwd_after_fwd(const hstu_layer_desc *desc, const hstu_layer_params *params,
                             const hstu_jagged *jagged, const void *x, const void *dy, void *dx,
                             const hstu_layer_grads *grads, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Action-oriented token embedding, "6.2. HSTU的工程突破" eq. 6.2.2:
 *   x[t] = item_emb[item_ids[t]] + action_emb[actions[t]]
 * item_emb [num_items, d], action_emb [num_actions, d], x [T, d] (dtype);
 * item_ids int64 [T], actions int32 [T] (device). A row whose id or action
 * is out of range is written as NaN (no out-of-bounds read). */
int hstu_embed_fwd(int64_t T, int32_t d_model, int32_t dtype, const void *item_emb,
                   int64_t num_items, const void *action_emb, int32_t num_actions,
                   const int64_t *item_ids, const int32_t *actions, void *x, void *stream);

/* Debug validation of device-resident index data (copies it to the host and
 * synchronises `stream`): offsets start at 0, do not decrease and end at T;
 * max_seq_len bounds every length; 0 <= num_targets[b] <= L_b; the cache
 * offsets likewise; every visible position difference fits the table; with
 * num_token_types > 1 every token type (own and cached) lies in
 * [0, num_token_types). Returns HSTU_OK or HSTU_E_DATA (with a message). */
int hstu_check_inputs(const hstu_layer_desc *desc, const hstu_jagged *jagged,
                      const hstu_kv_cache *cache, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
