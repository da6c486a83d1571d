// C ABI of the HSTU jagged layer forward: argument validation, workspace
// carving, dispatch to the gfx950 kernels and the layer composition
// (projection -> attention -> norm/gate -> f2 + residual). Every check runs
// on host scalars before anything is enqueued; no entry point allocates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/hstu.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return HSTU_OK;
}

}  // namespace

namespace hstu {

// The error channel for entry points implemented in other files.
int api_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void api_ok() { g_last_error.clear(); }

}  // namespace hstu

namespace {

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HSTU_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == HSTU_BF16 ? 2 : 4; }

#define CHECK(cond, code, ...)          \
  do {                                  \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_desc(const hstu_layer_desc* d) {
  CHECK(d != nullptr, HSTU_E_INVAL, "desc is NULL");
  CHECK(d->dtype == HSTU_F32 || d->dtype == HSTU_BF16, HSTU_E_INVAL, "unknown dtype %d", d->dtype);
  CHECK(d->num_heads > 0 && d->head_dim > 0, HSTU_E_INVAL, "num_heads and head_dim must be positive");
  CHECK(d->d_model == d->num_heads * d->head_dim, HSTU_E_INVAL,
        "d_model (%d) != num_heads (%d) * head_dim (%d)", d->d_model, d->num_heads, d->head_dim);
  if (d->dtype == HSTU_BF16) {
    CHECK(d->head_dim == 32 || d->head_dim == 64, HSTU_E_UNSUPPORTED,
          "bf16 supports head_dim 32 or 64 (got %d)", d->head_dim);
    CHECK(d->d_model <= 1024, HSTU_E_UNSUPPORTED, "d_model %d > 1024", d->d_model);
  } else {
    CHECK(d->head_dim == 32 || d->head_dim == 64, HSTU_E_UNSUPPORTED,
          "f32 supports head_dim 32 or 64 (got %d)", d->head_dim);
    CHECK(d->d_model <= 1024, HSTU_E_UNSUPPORTED, "d_model %d > 1024", d->d_model);
  }
  CHECK(std::isfinite(d->alpha) && std::fabs(d->alpha) >= 1e-6f && std::fabs(d->alpha) <= 1e6f,
        HSTU_E_INVAL, "alpha must satisfy 1e-6 <= |alpha| <= 1e6 (got %g)", d->alpha);
  CHECK(std::isfinite(d->ln_eps) && d->ln_eps >= 0.0f, HSTU_E_INVAL, "ln_eps must be finite and >= 0");
  CHECK(d->pos_table_len >= 1 && (d->pos_table_len & 1) == 1, HSTU_E_INVAL,
        "pos_table_len must be odd and positive (2*n_max-1), got %d", d->pos_table_len);
  CHECK(d->num_time_buckets >= 1 && d->num_time_buckets <= 64, HSTU_E_INVAL,
        "num_time_buckets must be in [1, 64] (got %d)", d->num_time_buckets);
  CHECK(d->input_norm == 0 || d->input_norm == 1, HSTU_E_INVAL, "input_norm must be 0 or 1 (got %d)",
        d->input_norm);
  CHECK(d->target_no_self == 0 || d->target_no_self == 1, HSTU_E_INVAL,
        "target_no_self must be 0 or 1 (got %d)", d->target_no_self);
  CHECK(d->num_token_types >= 0 && d->num_token_types <= HSTU_MAX_TOKEN_TYPES, HSTU_E_INVAL,
        "num_token_types must be in [0, %d] (got %d)", HSTU_MAX_TOKEN_TYPES, d->num_token_types);
  CHECK(d->bias_mode == HSTU_BIAS_TABLES || d->bias_mode == HSTU_BIAS_LINEAR, HSTU_E_INVAL,
        "unknown bias_mode %d", d->bias_mode);
  CHECK(d->attn_bwd_bf16 == 0 || d->attn_bwd_bf16 == 1, HSTU_E_INVAL, "attn_bwd_bf16 must be 0 or 1 (got %d)",
        d->attn_bwd_bf16);
  CHECK(d->gemm_bwd_bf16 == 0 || d->gemm_bwd_bf16 == 1, HSTU_E_INVAL, "gemm_bwd_bf16 must be 0 or 1 (got %d)",
        d->gemm_bwd_bf16);
  if (d->bias_mode == HSTU_BIAS_LINEAR) {
    CHECK(std::isfinite(d->linear_m_p) && std::isfinite(d->linear_m_t), HSTU_E_INVAL,
          "linear_m_p and linear_m_t must be finite");
    CHECK(d->num_token_types <= 1, HSTU_E_UNSUPPORTED,
          "the parameter-free bias has no token types (num_token_types %d)", d->num_token_types);
  }
  return HSTU_OK;
}

bool typed(const hstu_layer_desc* d) { return d->num_token_types > 1; }
bool linear_bias(const hstu_layer_desc* d) { return d->bias_mode == HSTU_BIAS_LINEAR; }

int check_jagged(const hstu_layer_desc* d, const hstu_jagged* j, const hstu_kv_cache* c) {
  CHECK(j != nullptr, HSTU_E_INVAL, "jagged is NULL");
  CHECK(j->num_seqs >= 0 && j->total_tokens >= 0 && j->max_seq_len >= 0, HSTU_E_INVAL,
        "negative jagged sizes");
  if (j->num_seqs > 0) CHECK(j->offsets != nullptr, HSTU_E_INVAL, "jagged offsets is NULL");
  if (j->total_tokens > 0) CHECK(j->timestamps != nullptr, HSTU_E_INVAL, "jagged timestamps is NULL");
  int64_t cache_max = 0;
  if (c) {
    CHECK(c->offsets != nullptr || j->num_seqs == 0, HSTU_E_INVAL, "cache offsets is NULL");
    CHECK(c->max_len >= 0 && c->total_tokens >= 0, HSTU_E_INVAL, "negative cache sizes");
    if (c->total_tokens > 0) {
      CHECK(c->k && c->v && c->timestamps, HSTU_E_INVAL, "cache k/v/timestamps is NULL");
      CHECK(aligned16(c->k) && aligned16(c->v), HSTU_E_INVAL, "cache k/v must be 16-byte aligned");
    }
    cache_max = c->max_len;
  }
  // Without targets the largest position difference is cache_len + L - 1,
  // bounded by the host scalars. With targets it depends on device data
  // (targets share one position); the kernels clamp table indices, and
  // hstu_check_inputs() checks the exact bound.
  if (typed(d)) {
    CHECK(j->total_tokens == 0 || j->token_types != nullptr, HSTU_E_INVAL,
          "jagged token_types is NULL with num_token_types %d", d->num_token_types);
    CHECK(!c || c->total_tokens == 0 || c->token_types != nullptr, HSTU_E_INVAL,
          "cache token_types is NULL with num_token_types %d", d->num_token_types);
  }
  const int64_t n_max = (static_cast<int64_t>(d->pos_table_len) + 1) / 2;
  if (j->num_targets == nullptr && !linear_bias(d))
    CHECK(static_cast<int64_t>(j->max_seq_len) + cache_max <= n_max, HSTU_E_INVAL,
          "position table too small: max_seq_len (%d) + cache max_len (%lld) > n_max (%lld)",
          j->max_seq_len, static_cast<long long>(cache_max), static_cast<long long>(n_max));
  return HSTU_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// The tiled bf16 attention kernel (work list, key-range splits, the fused
// norm_gate epilogue) takes head_dim 64; bf16 with head_dim 32 runs on the
// row-structured matrix-core kernel (plain causal) or the per-row kernel.
bool tiled_bf16(const hstu_layer_desc* d) { return d->dtype == HSTU_BF16 && d->head_dim == 64; }

hstu::AttnArgs make_attn_args(const hstu_layer_desc* d, const hstu_jagged* j,
                              const hstu_kv_cache* c, const void* q, const void* k,
                              const void* v, const float* pb, const float* tb, float* av,
                              void* ws, int max_splits = 8) {
  hstu::AttnArgs a{};
  a.sched = static_cast<int*>(ws);
  a.total_tokens = j->total_tokens;
  a.in_bf16 = d->dtype == HSTU_BF16 && !tiled_bf16(d);
  if (tiled_bf16(d)) {
    const hstu::AttnPlan plan = hstu::attn_plan(j->num_seqs, j->max_seq_len, d->num_heads, j->total_tokens,
                                                d->d_model, max_splits);
    a.bm = plan.bm;
    a.splits = plan.splits;
    a.partial = plan.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + plan.sched_bytes) : nullptr;
  } else {
    a.bm = 64;
    a.splits = 1;
    a.partial = nullptr;
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.ck = c ? c->k : nullptr;
  a.cv = c ? c->v : nullptr;
  a.offsets = j->offsets;
  a.ts = j->timestamps;
  a.num_targets = j->num_targets;
  a.no_self = d->target_no_self;
  a.c_offsets = c ? c->offsets : nullptr;
  a.c_ts = c ? c->timestamps : nullptr;
  a.pos_bias = pb;
  a.time_bias = tb;
  a.types = typed(d) ? j->token_types : nullptr;
  a.c_types = typed(d) && c ? c->token_types : nullptr;
  a.ntypes = typed(d) ? d->num_token_types : 1;
  a.linear = linear_bias(d) ? 1 : 0;
  a.m_p = d->linear_m_p;
  a.m_t = d->linear_m_t;
  a.av = av;
  a.d_model = d->d_model;
  a.num_heads = d->num_heads;
  a.head_dim = d->head_dim;
  a.pos_len = d->pos_table_len;
  a.pos_center = (d->pos_table_len - 1) / 2;
  a.nb = d->num_time_buckets;
  a.alpha = d->alpha;
  a.num_seqs = j->num_seqs;
  a.max_seq_len = j->max_seq_len;
  a.max_cache_len = c ? c->max_len : 0;
  return a;
}

int do_proj(const hstu_layer_desc* d, const hstu_layer_params* p, int64_t T, const void* x,
            void* u, void* v, void* q, void* k, hipStream_t s, const hstu::AttnArgs* sched = nullptr) {
  hstu::ProjArgs a{};
  a.sched = sched;
  a.x = x;
  a.w = p->w1;
  a.bias = p->b1;
  a.out[0] = u;
  a.out[1] = v;
  a.out[2] = q;
  a.out[3] = k;
  a.M = T;
  a.K = d->d_model;
  return device_status(d->dtype == HSTU_BF16 ? hstu::launch_proj_bf16(a, s) : hstu::launch_proj_f32(a, s),
                       "proj launch");
}

hstu::BwdAttnArgs make_train_args(const hstu_layer_desc* d, const hstu_jagged* j, const float* q,
                                  const float* k, const float* v, const float* pb, const float* tb) {
  hstu::BwdAttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.offsets = j->offsets; a.ts = j->timestamps;
  a.pos_bias = pb; a.time_bias = tb;
  a.d_model = d->d_model; a.num_heads = d->num_heads; a.head_dim = d->head_dim;
  a.pos_len = d->pos_table_len; a.pos_center = (d->pos_table_len - 1) / 2;
  a.nb = d->num_time_buckets; a.alpha = d->alpha;
  a.num_seqs = j->num_seqs; a.max_seq_len = j->max_seq_len;
  return a;
}

int do_attn(const hstu_layer_desc* d, const hstu_jagged* j, const hstu_kv_cache* c, const void* q,
            const void* k, const void* v, const float* pb, const float* tb, float* av, void* ws,
            hipStream_t s, int max_splits = 8) {
  if (d->dtype == HSTU_F32 && c == nullptr && j->num_targets == nullptr && !typed(d) && !linear_bias(d) &&
      hstu::attn_train_supported(d->head_dim) &&
      static_cast<int64_t>(j->max_seq_len) * d->d_model < (int64_t{1} << 31)) {
    // plain causal fp32: the matrix-core kernel
    hstu::BwdAttnArgs ta = make_train_args(d, j, static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), pb, tb);
    ta.av = av;
    return device_status(hstu::launch_attn_train_fwd(ta, s), "attention launch");
  }
  if (d->dtype == HSTU_BF16 && !tiled_bf16(d) && c == nullptr && j->num_targets == nullptr && !typed(d) &&
      !linear_bias(d) && static_cast<int64_t>(j->max_seq_len) * d->d_model < (int64_t{1} << 31)) {
    // plain causal bf16 with head_dim 32: the row-structured matrix-core kernel
    hstu::BwdAttnArgs ta = make_train_args(d, j, nullptr, nullptr, nullptr, pb, tb);
    ta.q16 = static_cast<const uint16_t*>(q);
    ta.k16 = static_cast<const uint16_t*>(k);
    ta.v16 = static_cast<const uint16_t*>(v);
    ta.av = av;
    return device_status(hstu::launch_attn_fwd_bf16_rows(ta, s), "attention launch");
  }
  const hstu::AttnArgs a = make_attn_args(d, j, c, q, k, v, pb, tb, av, ws, max_splits);
  return device_status(tiled_bf16(d) ? hstu::launch_attn_bf16(a, s) : hstu::launch_attn_f32(a, s),
                       "attention launch");
}

int do_norm_gate(const hstu_layer_desc* d, int64_t T, const float* av, const void* u,
                 const float* gamma, const float* beta, void* g, hipStream_t s) {
  hstu::NormGateArgs a{av, u, gamma, beta, g, T, d->d_model, d->ln_eps};
  return device_status(d->dtype == HSTU_BF16 ? hstu::launch_norm_gate_bf16(a, s)
                                             : hstu::launch_norm_gate_f32(a, s),
                       "norm_gate launch");
}

int do_layernorm(const hstu_layer_desc* d, int64_t T, const void* x, const float* gamma,
                 const float* beta, void* y, hipStream_t s) {
  hstu::LayerNormArgs a{x, gamma, beta, y, T, d->d_model, d->ln_eps};
  return device_status(d->dtype == HSTU_BF16 ? hstu::launch_layernorm_bf16(a, s)
                                             : hstu::launch_layernorm_f32(a, s),
                       "layernorm launch");
}

int do_out(const hstu_layer_desc* d, int64_t T, const void* g, const void* x, const void* w2,
           const float* b2, void* y, hipStream_t s) {
  hstu::OutArgs a{g, w2, b2, x, y, T, d->d_model};
  return device_status(d->dtype == HSTU_BF16 ? hstu::launch_out_bf16(a, s) : hstu::launch_out_f32(a, s),
                       "out launch");
}

size_t round256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

size_t attn_ws(const hstu_layer_desc* d, const hstu_jagged* j) {
  if (!tiled_bf16(d) || j->num_seqs <= 0 || j->max_seq_len <= 0) return 0;
  return round256(
      hstu::attn_plan(j->num_seqs, j->max_seq_len, d->num_heads, j->total_tokens, d->d_model).workspace_bytes);
}

// the work list indexes (item, key chunk) units, item = seq * n_tiles + tile,
// in int32
int check_items(const hstu_jagged* j) {
  const int64_t n_qt = (static_cast<int64_t>(j->max_seq_len) + 63) / 64;
  CHECK(static_cast<int64_t>(j->num_seqs) * n_qt * 8 < (int64_t{1} << 31) - 1, HSTU_E_UNSUPPORTED,
        "num_seqs * ceil(max_seq_len / 64) must stay below 2^28");
  return HSTU_OK;
}

}  // namespace

extern "C" {

int hstu_abi_version(void) { return HSTU_ABI_VERSION; }

const char* hstu_last_error(void) { return g_last_error.c_str(); }

int hstu_proj_fwd(const hstu_layer_desc* desc, const hstu_layer_params* params, int64_t T,
                  const void* x, void* u, void* v, void* q, void* k, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  CHECK(params != nullptr && params->w1 != nullptr, HSTU_E_INVAL, "params or w1 is NULL");
  CHECK(T >= 0, HSTU_E_INVAL, "T must be >= 0");
  if (T == 0) return ok();
  CHECK(x && u && v && q && k, HSTU_E_INVAL, "x/u/v/q/k must not be NULL");
  CHECK(aligned16(x) && aligned16(u) && aligned16(v) && aligned16(q) && aligned16(k) &&
            aligned16(params->w1),
        HSTU_E_INVAL, "activations and w1 must be 16-byte aligned");
  return do_proj(desc, params, T, x, u, v, q, k, as_stream(stream));
}

size_t hstu_attn_workspace_size(const hstu_layer_desc* desc, const hstu_jagged* jagged) {
  if (!desc || !jagged) return 0;
  return attn_ws(desc, jagged);
}

int hstu_attn_fwd(const hstu_layer_desc* desc, const hstu_jagged* jagged,
                  const hstu_kv_cache* cache, const void* q, const void* k, const void* v,
                  const float* pos_bias, const float* time_bias, float* av, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  st = check_jagged(desc, jagged, cache);
  if (st) return st;
  st = check_items(jagged);
  if (st) return st;
  if (jagged->num_seqs == 0 || jagged->total_tokens == 0) return ok();
  CHECK(q && k && v && av, HSTU_E_INVAL, "q/k/v/av must not be NULL");
  CHECK(linear_bias(desc) || (pos_bias && time_bias), HSTU_E_INVAL, "pos_bias/time_bias must not be NULL");
  CHECK(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(av), HSTU_E_INVAL,
        "q/k/v/av must be 16-byte aligned");
  const size_t need = attn_ws(desc, jagged);
  CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), HSTU_E_WORKSPACE,
        "workspace too small: need %zu bytes, got %zu", need, workspace_bytes);
  CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HSTU_E_INVAL,
        "workspace must be 256-byte aligned");
  return do_attn(desc, jagged, cache, q, k, v, pos_bias, time_bias, av, workspace,
                 as_stream(stream));
}

int hstu_attn_fwd_noalloc(const hstu_layer_desc* desc, const hstu_jagged* jagged,
                          const hstu_kv_cache* cache, const void* q, const void* k, const void* v,
                          const float* pos_bias, const float* time_bias, float* av, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  st = check_jagged(desc, jagged, cache);
  if (st) return st;
  st = check_items(jagged);
  if (st) return st;
  if (jagged->num_seqs == 0 || jagged->total_tokens == 0) return ok();
  CHECK(q && k && v && av, HSTU_E_INVAL, "q/k/v/av must not be NULL");
  CHECK(linear_bias(desc) || (pos_bias && time_bias), HSTU_E_INVAL, "pos_bias/time_bias must not be NULL");
  CHECK(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(av), HSTU_E_INVAL,
        "q/k/v/av must be 16-byte aligned");
  void* ws = nullptr;
  int max_splits = 8;
  if (tiled_bf16(desc)) {
    // the most key-range splits whose work list and partial outputs fit the
    // static scratch (fewer splits only change the order of the fp32 sums)
    const size_t cap = hstu::kAttnStaticScratchBytes;
    for (;;) {
      const hstu::AttnPlan p = hstu::attn_plan(jagged->num_seqs, jagged->max_seq_len, desc->num_heads,
                                               jagged->total_tokens, desc->d_model, max_splits);
      if (p.workspace_bytes <= cap) break;
      CHECK(p.splits > 1, HSTU_E_WORKSPACE,
            "batch too large for the static scratch: its work list needs %zu bytes, the scratch holds %zu",
            p.workspace_bytes, cap);
      max_splits = p.splits - 1;
    }
    CHECK(hstu::attn_static_scratch(&ws) == hipSuccess, HSTU_E_DEVICE,
          "could not resolve the static scratch on the current device");
  }
  return do_attn(desc, jagged, cache, q, k, v, pos_bias, time_bias, av, ws, as_stream(stream), max_splits);
}

int hstu_norm_gate_fwd(const hstu_layer_desc* desc, int64_t T, const float* av, const void* u,
                       const float* gamma, const float* beta, void* g, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  CHECK(T >= 0, HSTU_E_INVAL, "T must be >= 0");
  if (T == 0) return ok();
  CHECK(av && u && g, HSTU_E_INVAL, "av/u/g must not be NULL");
  CHECK(aligned16(av) && aligned16(u) && aligned16(g), HSTU_E_INVAL, "av/u/g must be 16-byte aligned");
  CHECK(!gamma || aligned16(gamma), HSTU_E_INVAL, "gamma must be 16-byte aligned");
  CHECK(!beta || aligned16(beta), HSTU_E_INVAL, "beta must be 16-byte aligned");
  return do_norm_gate(desc, T, av, u, gamma, beta, g, as_stream(stream));
}

int hstu_layernorm_fwd(const hstu_layer_desc* desc, int64_t T, const void* x, const float* gamma,
                       const float* beta, void* y, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  CHECK(T >= 0, HSTU_E_INVAL, "T must be >= 0");
  if (T == 0) return ok();
  CHECK(x && y, HSTU_E_INVAL, "x/y must not be NULL");
  CHECK(x != y, HSTU_E_INVAL, "y must not alias x");
  CHECK(aligned16(x) && aligned16(y), HSTU_E_INVAL, "x/y must be 16-byte aligned");
  CHECK(!gamma || aligned16(gamma), HSTU_E_INVAL, "gamma must be 16-byte aligned");
  CHECK(!beta || aligned16(beta), HSTU_E_INVAL, "beta must be 16-byte aligned");
  return do_layernorm(desc, T, x, gamma, beta, y, as_stream(stream));
}

int hstu_linear_bias_tables(const hstu_layer_desc* desc, float m_p, float m_t, float* pos_bias,
                            float* time_bias, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  CHECK(std::isfinite(m_p) && std::isfinite(m_t), HSTU_E_INVAL, "m_p and m_t must be finite");
  CHECK(pos_bias && time_bias, HSTU_E_INVAL, "pos_bias/time_bias must not be NULL");
  CHECK(pos_bias != time_bias, HSTU_E_INVAL, "pos_bias and time_bias must not alias");
  const int pairs = typed(desc) ? desc->num_token_types * desc->num_token_types : 1;
  return device_status(hstu::launch_linear_bias_tables(m_p, m_t, desc->pos_table_len,
                                                       desc->num_time_buckets, pairs, pos_bias, time_bias,
                                                       as_stream(stream)),
                       "linear bias tables launch");
}

int hstu_gather_rows(int64_t n, int32_t row_bytes, const int64_t* rows, int64_t src_rows,
                     const void* src, void* dst, void* stream) {
  CHECK(n >= 0 && src_rows >= 0, HSTU_E_INVAL, "n and src_rows must be >= 0");
  CHECK(row_bytes > 0 && row_bytes % 8 == 0, HSTU_E_INVAL, "row_bytes must be a positive multiple of 8");
  if (n == 0) return ok();
  CHECK(src_rows > 0, HSTU_E_INVAL, "gathering from an empty source");
  CHECK(rows && src && dst, HSTU_E_INVAL, "rows/src/dst must not be NULL");
  CHECK((reinterpret_cast<uintptr_t>(src) & 7u) == 0 && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0,
        HSTU_E_INVAL, "src/dst must be 8-byte aligned");
  CHECK(src != dst, HSTU_E_INVAL, "dst must not alias src");
  return device_status(hstu::launch_gather_rows(n, row_bytes, rows, src_rows, src, dst, as_stream(stream)),
                       "gather launch");
}

int hstu_kv_cache_concat(const hstu_layer_desc* desc, int32_t num_seqs, const hstu_kv_cache* a,
                         const hstu_kv_cache* n, int64_t* out_offsets, int64_t* out_timestamps,
                         void* out_k, void* out_v, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  CHECK(num_seqs >= 0, HSTU_E_INVAL, "num_seqs must be >= 0");
  CHECK(a && n, HSTU_E_INVAL, "a and n must not be NULL");
  CHECK(a->total_tokens >= 0 && n->total_tokens >= 0, HSTU_E_INVAL, "total_tokens must be >= 0");
  CHECK(a->offsets && n->offsets && out_offsets, HSTU_E_INVAL, "offsets must not be NULL");
  const int64_t rows = a->total_tokens + n->total_tokens;
  CHECK(num_seqs > 0 || rows == 0, HSTU_E_INVAL, "rows without sequences");
  if (rows > 0) {
    CHECK(out_timestamps && out_k && out_v, HSTU_E_INVAL, "outputs must not be NULL");
    CHECK(aligned16(out_k) && aligned16(out_v), HSTU_E_INVAL, "out_k/out_v must be 16-byte aligned");
    for (const hstu_kv_cache* c : {a, n}) {
      if (c->total_tokens == 0) continue;
      CHECK(c->timestamps && c->k && c->v, HSTU_E_INVAL, "cache timestamps/k/v must not be NULL");
      CHECK(aligned16(c->k) && aligned16(c->v), HSTU_E_INVAL, "cache k/v must be 16-byte aligned");
      CHECK(c->k != out_k && c->k != out_v && c->v != out_k && c->v != out_v &&
                c->timestamps != out_timestamps && c->offsets != out_offsets,
            HSTU_E_INVAL, "outputs must not alias the inputs");
    }
  }
  const int row_bytes = desc->d_model * static_cast<int>(elem_size(desc->dtype));
  hstu::CacheConcatArgs c{a->offsets, a->timestamps, a->k, a->v,
                          n->offsets, n->timestamps, n->k, n->v,
                          out_offsets, out_timestamps, out_k, out_v,
                          rows, a->total_tokens, n->total_tokens, num_seqs, row_bytes};
  return device_status(hstu::launch_cache_concat(c, as_stream(stream)), "cache concat launch");
}

int hstu_out_fwd(const hstu_layer_desc* desc, int64_t T, const void* g, const void* x,
                 const void* w2, const float* b2, void* y, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  CHECK(T >= 0, HSTU_E_INVAL, "T must be >= 0");
  if (T == 0) return ok();
  CHECK(g && x && w2 && y, HSTU_E_INVAL, "g/x/w2/y must not be NULL");
  CHECK(aligned16(g) && aligned16(x) && aligned16(w2) && aligned16(y), HSTU_E_INVAL,
        "g/x/w2/y must be 16-byte aligned");
  CHECK(y != x && y != g, HSTU_E_INVAL, "y must not alias x or g");
  return do_out(desc, T, g, x, w2, b2, y, as_stream(stream));
}

size_t hstu_layer_workspace_size(const hstu_layer_desc* desc, const hstu_jagged* jagged) {
  if (!desc || !jagged || jagged->total_tokens < 0 || desc->d_model <= 0) return 0;
  const size_t T = static_cast<size_t>(jagged->total_tokens);
  const size_t act = round256(T * desc->d_model * elem_size(desc->dtype));
  const size_t av = round256(T * desc->d_model * sizeof(float));
  // U, V, Q, K (G overwrites U), AV, work list, then LayerNorm(X) with input_norm
  return 4 * act + av + attn_ws(desc, jagged) + (desc->input_norm ? act : 0);
}

int hstu_layer_fwd(const hstu_layer_desc* desc, const hstu_layer_params* params,
                   const hstu_jagged* jagged, const hstu_kv_cache* cache, const void* x, void* y,
                   void* k_out, void* v_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  st = check_jagged(desc, jagged, cache);
  if (st) return st;
  CHECK(params && params->w1 && params->w2 && (linear_bias(desc) || (params->pos_bias && params->time_bias)),
        HSTU_E_INVAL, "params, w1, w2, pos_bias and time_bias must not be NULL");
  st = check_items(jagged);
  if (st) return st;
  const int64_t T = jagged->total_tokens;
  if (T == 0 || jagged->num_seqs == 0) return ok();
  CHECK(x && y, HSTU_E_INVAL, "x/y must not be NULL");
  CHECK(x != y, HSTU_E_INVAL, "y must not alias x");
  CHECK(aligned16(x) && aligned16(y) && aligned16(params->w1) && aligned16(params->w2),
        HSTU_E_INVAL, "x/y/w1/w2 must be 16-byte aligned");
  CHECK((!k_out || aligned16(k_out)) && (!v_out || aligned16(v_out)), HSTU_E_INVAL,
        "k_out/v_out must be 16-byte aligned");
  CHECK(!params->ln_gamma || aligned16(params->ln_gamma), HSTU_E_INVAL, "ln_gamma must be 16-byte aligned");
  CHECK(!params->ln_beta || aligned16(params->ln_beta), HSTU_E_INVAL, "ln_beta must be 16-byte aligned");
  CHECK(!desc->input_norm || ((!params->ln1_gamma || aligned16(params->ln1_gamma)) &&
                              (!params->ln1_beta || aligned16(params->ln1_beta))),
        HSTU_E_INVAL, "ln1_gamma/ln1_beta must be 16-byte aligned");
  const size_t need = hstu_layer_workspace_size(desc, jagged);
  CHECK(workspace != nullptr && workspace_bytes >= need, HSTU_E_WORKSPACE,
        "workspace too small: need %zu bytes, got %zu", need, workspace_bytes);
  CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HSTU_E_INVAL,
        "workspace must be 256-byte aligned");
  const size_t act = round256(static_cast<size_t>(T) * desc->d_model * elem_size(desc->dtype));
  char* ws = static_cast<char*>(workspace);
  void* u = ws;
  void* v = ws + act;
  void* q = ws + 2 * act;
  void* k = ws + 3 * act;
  float* av = reinterpret_cast<float*>(ws + 4 * act);
  void* attn_work = ws + 4 * act + round256(static_cast<size_t>(T) * desc->d_model * sizeof(float));
  if (k_out) k = k_out;
  if (v_out) v = v_out;
  hipStream_t s = as_stream(stream);
  const void* xin = x;   // what f1 reads; the residual below always adds the raw x
  if (desc->input_norm) {
    void* xn = ws + 4 * act + round256(static_cast<size_t>(T) * desc->d_model * sizeof(float)) +
               attn_ws(desc, jagged);
    st = do_layernorm(desc, T, x, params->ln1_gamma, params->ln1_beta, xn, s);
    if (st) return st;
    xin = xn;
  }
  if (tiled_bf16(desc) &&
      hstu::attn_can_fuse_norm_gate(jagged->num_seqs, jagged->max_seq_len, desc->num_heads, jagged->total_tokens,
                                    desc->d_model)) {
    // one head group covers each row: the attention kernel finishes the rows
    // into G = norm_gate(AV, U) itself (in place over U), with the same row
    // code as hstu_norm_gate_fwd, so Y is bitwise that of the separate calls.
    // Its work list comes from one extra workgroup of the f1 launch.
    hstu::AttnArgs a = make_attn_args(desc, jagged, cache, q, k, v, params->pos_bias, params->time_bias, av,
                                      attn_work);
    a.fuse_ng = 1;
    a.ng_u = u;
    a.ng_g = u;
    a.ng_gamma = params->ln_gamma;
    a.ng_beta = params->ln_beta;
    a.ng_eps = desc->ln_eps;
    st = do_proj(desc, params, T, xin, u, v, q, k, s, &a);
    if (st) return st;
    a.sched_ready = 1;
    st = device_status(hstu::launch_attn_bf16(a, s), "attention launch");
  } else {
    st = do_proj(desc, params, T, xin, u, v, q, k, s);
    if (st) return st;
    st = do_attn(desc, jagged, cache, q, k, v, params->pos_bias, params->time_bias, av, attn_work, s);
    if (st) return st;
    st = do_norm_gate(desc, T, av, u, params->ln_gamma, params->ln_beta, u, s);
  }
  if (st) return st;
  return do_out(desc, T, u, x, params->w2, params->b2, y, s);
}

namespace {

// The weight gradients of the bf16 backward contract over the T tokens: S
// splits of kc tokens each (kc % 32 == 0), the transposed operand copies
// zero-padded to tp = S * kc columns. Up to 32 splits, so that a product with
// 16 to 32 output tiles fills the chip.
struct TokSplit {
  int S;
  int kc;
  int64_t tp;
};
TokSplit tok_split(int64_t T) {
  const int64_t steps = std::max<int64_t>(1, (T + 31) / 32);
  const int64_t S = std::min<int64_t>(32, steps);
  const int64_t kc = (steps + S - 1) / S * 32;
  return {static_cast<int>(S), static_cast<int>(kc), S * kc};
}

// Byte offsets of the bf16 products' buffers, from the start of their
// region: the operands of f1 as bf16 hi/lo splits (Xin [T, 3d], W1 [4d, 3d]),
// those of f2 (G, W2) in bf16; dY and dZ in
// bf16; dY^T, G^T, Xin^T and dZ^T in bf16 with tp columns; W1^T and W2^T in
// bf16; the split partial sums of dW1 or dW2.
struct GemmBf16Ws {
  size_t xin16, w1_16, g16, w2_16, dy16, dz16, dyt, gt, xint, dzt, w1t, w2t, part, bytes;
};
GemmBf16Ws gemm_bf16_ws(int64_t T, int d) {
  const TokSplit ts = tok_split(T);
  const size_t t = static_cast<size_t>(T), dd = static_cast<size_t>(d), tp = static_cast<size_t>(ts.tp);
  GemmBf16Ws w{};
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += round256(n);
    return at;
  };
  w.xin16 = take(t * 3 * dd * 2);
  w.w1_16 = take(4 * dd * 3 * dd * 2);
  w.g16 = take(t * dd * 2);
  w.w2_16 = take(dd * dd * 2);
  w.dy16 = take(t * dd * 2);
  w.dz16 = take(t * 4 * dd * 2);
  w.dyt = take(dd * tp * 2);
  w.gt = take(dd * tp * 2);
  w.xint = take(dd * tp * 2);
  w.dzt = take(4 * dd * tp * 2);
  w.w1t = take(4 * dd * dd * 2);
  w.w2t = take(dd * dd * 2);
  w.part = take(static_cast<size_t>(ts.S) * 4 * dd * dd * 4);
  w.bytes = o;
  return w;
}

// Bytes of the fp32 layout and the bf16 attention copies: where the bf16
// products' region starts.
size_t train_ws_base(const hstu_layer_desc* desc, size_t T) {
  const size_t td = round256(T * desc->d_model * sizeof(float));
  // with the bf16 attention backward: bf16 copies of Q, K, V and dAV
  const size_t bf = desc->attn_bwd_bf16 == 1 ? 4 * round256(T * desc->d_model * sizeof(uint16_t)) : 0;
  return (desc->input_norm ? 18 : 17) * td + round256(T * sizeof(float)) + bf;
}

// With attn_bwd_bf16 the attention forward of the training layer also runs
// on bf16 (from the bf16 copies of Q, K, V): head_dim 64 on the tiled kernel,
// whose work list and partial outputs follow the bf16 products' region, and
// head_dim 32 on the row-structured kernel, which needs no workspace.
bool train_fwd_bf16(const hstu_layer_desc* desc) {
  return desc->attn_bwd_bf16 == 1 && desc->head_dim == 64 && desc->d_model <= 1024;
}
size_t train_attn16_bytes(const hstu_layer_desc* desc, const hstu_jagged* j) {
  if (!train_fwd_bf16(desc)) return 0;
  return round256(hstu::attn_plan(j->num_seqs, j->max_seq_len, desc->num_heads, j->total_tokens,
                                  desc->d_model).workspace_bytes);
}

}  // namespace

size_t hstu_layer_bwd_workspace_size(const hstu_layer_desc* desc, const hstu_jagged* jagged) {
  if (!desc || !jagged || jagged->total_tokens < 0 || desc->d_model <= 0 || jagged->num_seqs < 0 ||
      jagged->max_seq_len < 0)
    return 0;
  const size_t T = static_cast<size_t>(jagged->total_tokens);
  const size_t g16 = desc->gemm_bwd_bf16 == 1 ? gemm_bf16_ws(jagged->total_tokens, desc->d_model).bytes : 0;
  return train_ws_base(desc, T) + g16 + train_attn16_bytes(desc, jagged);
}

namespace {

// The fp32 training layer. kTrainFull: forward recompute, then the backward
// (hstu_layer_bwd). kTrainForward: the forward with Y, keeping in the
// workspace what the backward reads (hstu_layer_fwd_train). kTrainBackward:
// the backward from such a workspace (hstu_layer_bwd_after_fwd).
enum { kTrainFull = 0, kTrainForward = 1, kTrainBackward = 2 };

int layer_train(const hstu_layer_desc* desc, const hstu_layer_params* params, const hstu_jagged* jagged,
                const void* x, const void* dy, void* dx, void* y, const hstu_layer_grads* grads,
                void* workspace, size_t workspace_bytes, void* stream, int mode) {
  const bool fwd = mode != kTrainBackward, bwd = mode != kTrainForward;
  int st = check_desc(desc);
  if (st) return st;
  CHECK(desc->dtype == HSTU_F32, HSTU_E_UNSUPPORTED, "the backward pass supports dtype f32");
  st = check_jagged(desc, jagged, nullptr);
  if (st) return st;
  CHECK(jagged->num_targets == nullptr, HSTU_E_UNSUPPORTED,
        "the backward pass supports plain causal attention (no targets)");
  CHECK(!typed(desc) && !linear_bias(desc), HSTU_E_UNSUPPORTED,
        "the backward pass supports the untyped table bias");
  CHECK(jagged->total_tokens < (int64_t{1} << 31) &&
            static_cast<int64_t>(jagged->max_seq_len) * desc->d_model < (int64_t{1} << 31),
        HSTU_E_UNSUPPORTED, "the backward pass needs total_tokens and max_seq_len * d_model below 2^31");
  CHECK(params && params->w1 && params->w2 && params->pos_bias && params->time_bias, HSTU_E_INVAL,
        "params, w1, w2, pos_bias and time_bias must not be NULL");
  CHECK(!bwd || (grads && grads->dw1 && grads->db1 && grads->dw2 && grads->db2 && grads->dgamma &&
                  grads->dbeta && grads->dpos && grads->dtime),
        HSTU_E_INVAL, "every gradient pointer must be set");
  const bool norm1 = desc->input_norm != 0;
  CHECK(!bwd || !norm1 || (grads->dln1_gamma && grads->dln1_beta), HSTU_E_INVAL,
        "with input_norm, dln1_gamma and dln1_beta must be set");
  CHECK(!norm1 || ((!params->ln1_gamma || aligned16(params->ln1_gamma)) &&
                   (!params->ln1_beta || aligned16(params->ln1_beta))),
        HSTU_E_INVAL, "ln1_gamma/ln1_beta must be 16-byte aligned");
  CHECK((!params->ln_gamma || aligned16(params->ln_gamma)) && (!params->ln_beta || aligned16(params->ln_beta)),
        HSTU_E_INVAL, "ln_gamma/ln_beta must be 16-byte aligned");
  const int64_t T = jagged->total_tokens;
  const int d = desc->d_model;
  const bool empty = T == 0 || jagged->num_seqs == 0;
  if (!empty) {
    if (bwd) {
      CHECK(x && dy && dx, HSTU_E_INVAL, "x/dy/dx must not be NULL");
      CHECK(dx != x && dx != dy, HSTU_E_INVAL, "dx must not alias x or dy");
      CHECK(aligned16(x) && aligned16(dy) && aligned16(dx), HSTU_E_INVAL,
            "x/dy/dx must be 16-byte aligned");
    } else {
      CHECK(x && y, HSTU_E_INVAL, "x/y must not be NULL");
      CHECK(y != x, HSTU_E_INVAL, "y must not alias x");
      CHECK(aligned16(x) && aligned16(y), HSTU_E_INVAL, "x/y must be 16-byte aligned");
    }
    const size_t need = hstu_layer_bwd_workspace_size(desc, jagged);
    CHECK(workspace != nullptr && workspace_bytes >= need, HSTU_E_WORKSPACE,
          "workspace too small: need %zu bytes, got %zu", need, workspace_bytes);
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HSTU_E_INVAL,
          "workspace must be 256-byte aligned");
  }
  hipStream_t s = as_stream(stream);
  if (bwd) {
    // gradients start at zero (also for an empty batch), in one launch
    const struct { float* p; int64_t n; } zero[] = {
        {grads->dw1, 4LL * d * d}, {grads->db1, 4LL * d}, {grads->dw2, 1LL * d * d}, {grads->db2, d},
        {grads->dgamma, d}, {grads->dbeta, d}, {grads->dpos, desc->pos_table_len},
        {grads->dtime, desc->num_time_buckets},
        {norm1 ? grads->dln1_gamma : nullptr, norm1 ? d : 0},
        {norm1 ? grads->dln1_beta : nullptr, norm1 ? d : 0}};
    static_assert(sizeof(zero) / sizeof(zero[0]) <= hstu::kZeroListMax, "zero list");
    hstu::ZeroList zl{};
    for (const auto& z : zero) {
      if (z.n == 0) continue;
      zl.p[zl.count] = z.p;
      zl.n[zl.count] = z.n;
      ++zl.count;
    }
    st = device_status(hstu::launch_fill_zero_list(zl, s), "zero fill");
    if (st) return st;
  }
  if (empty) return ok();
  const size_t td = round256(static_cast<size_t>(T) * d * sizeof(float));
  char* w = static_cast<char*>(workspace);
  float* Z = reinterpret_cast<float*>(w);             // [T, 4d] pre-activation
  float* U = reinterpret_cast<float*>(w + 4 * td);
  float* V = reinterpret_cast<float*>(w + 5 * td);
  float* Q = reinterpret_cast<float*>(w + 6 * td);
  float* K = reinterpret_cast<float*>(w + 7 * td);
  float* AV = reinterpret_cast<float*>(w + 8 * td);
  float* NH = reinterpret_cast<float*>(w + 9 * td);
  float* G = reinterpret_cast<float*>(w + 10 * td);
  float* DG = reinterpret_cast<float*>(w + 11 * td);
  float* DZ = reinterpret_cast<float*>(w + 12 * td);   // [T, 4d]: dU, dV, dQ, dK
  float* DAV = reinterpret_cast<float*>(w + 16 * td);
  float* RSTD = reinterpret_cast<float*>(w + 17 * td);
  // LayerNorm(X) with input_norm: the input of f1
  float* XN = norm1 ? reinterpret_cast<float*>(w + 17 * td + round256(static_cast<size_t>(T) * sizeof(float)))
                    : nullptr;
  // bf16 copies of Q, K, V, dAV for the bf16 attention backward
  const bool bf16_bwd = desc->attn_bwd_bf16 == 1;
  const size_t tb16 = round256(static_cast<size_t>(T) * d * sizeof(uint16_t));
  uint16_t* B16 = reinterpret_cast<uint16_t*>(w + (norm1 ? 18 : 17) * td +
                                              round256(static_cast<size_t>(T) * sizeof(float)));
  uint16_t* Q16 = B16;
  uint16_t* K16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(B16) + tb16);
  uint16_t* V16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(B16) + 2 * tb16);
  uint16_t* DAV16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(B16) + 3 * tb16);

  // the attention forward on the bf16 kernel: its work list and partials
  const bool fwd16 = train_fwd_bf16(desc);
  void* const attn16_ws = w + train_ws_base(desc, static_cast<size_t>(T)) +
                          (desc->gemm_bwd_bf16 == 1 ? gemm_bf16_ws(T, d).bytes : 0);
  // bf16 operand copies and split partials of the backward's products
  const bool g16 = desc->gemm_bwd_bf16 == 1;
  const TokSplit ts = tok_split(T);
  const GemmBf16Ws gw = gemm_bf16_ws(T, d);
  char* const g16w = w + train_ws_base(desc, static_cast<size_t>(T));
  uint16_t* const XIN16 = reinterpret_cast<uint16_t*>(g16w + gw.xin16);
  uint16_t* const W1_16 = reinterpret_cast<uint16_t*>(g16w + gw.w1_16);
  uint16_t* const G16 = reinterpret_cast<uint16_t*>(g16w + gw.g16);
  uint16_t* const W2_16 = reinterpret_cast<uint16_t*>(g16w + gw.w2_16);
  uint16_t* const DY16 = reinterpret_cast<uint16_t*>(g16w + gw.dy16);
  uint16_t* const DZ16 = reinterpret_cast<uint16_t*>(g16w + gw.dz16);
  uint16_t* const DYT = reinterpret_cast<uint16_t*>(g16w + gw.dyt);
  uint16_t* const GT = reinterpret_cast<uint16_t*>(g16w + gw.gt);
  uint16_t* const XINT = reinterpret_cast<uint16_t*>(g16w + gw.xint);
  uint16_t* const DZT = reinterpret_cast<uint16_t*>(g16w + gw.dzt);
  uint16_t* const W1T = reinterpret_cast<uint16_t*>(g16w + gw.w1t);
  uint16_t* const W2T = reinterpret_cast<uint16_t*>(g16w + gw.w2t);
  float* const PART = reinterpret_cast<float*>(g16w + gw.part);

  const float* X = static_cast<const float*>(x);
  const float* DY = static_cast<const float*>(dy);
  const float* W1 = static_cast<const float*>(params->w1);
  const float* W2 = static_cast<const float*>(params->w2);
  const int d4 = 4 * d;
  // weight gradients reduce over T: split it so that the grid has ~2048 blocks
  auto splits = [&](int M, int N) {
    const int64_t tiles = static_cast<int64_t>((M + 63) / 64) * ((N + 63) / 64);
    const int64_t sp = (2048 + tiles - 1) / tiles;
    const int64_t cap = (T + 255) / 256;
    return static_cast<int>(std::max<int64_t>(1, std::min(sp, cap)));
  };
#define HSTU_TRY(expr, what)                       \
  do {                                             \
    st = device_status((expr), what);              \
    if (st) return st;                             \
  } while (0)
  hstu::BwdAttnArgs ba = make_train_args(desc, jagged, Q, K, V, params->pos_bias, params->time_bias);
  ba.av = AV;
  const float* XIN = norm1 ? XN : X;   // the input of f1
  // C[M, N] = A[M, K] B[N, K]^T on bf16 copies (K = S * kc with splits)
  auto gemm16 = [&](const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, float* c, int64_t ldc,
                    const float* addend, int64_t M, int N, int kc, int S) {
    hstu::GemmBf16Args g{a, lda, b, ldb, c, ldc, addend, M, N, kc, S};
    return hstu::launch_gemm_bf16_f32(g, s);
  };
  // forward: Z = X W1^T + b1 and [U V Q K] = SiLU(Z) in one pass
  if (fwd) {
    if (norm1) {
      st = do_layernorm(desc, T, x, params->ln1_gamma, params->ln1_beta, XN, s);
      if (st) return st;
    }
  }
  if (fwd && g16) {
    // f1 feeds every gradient: its operands are split into bf16 hi and lo
    // parts, [Xh | Xl | Xh] [Wh | Wh | Wl]^T over 3d, fp32-like products
    // (the same pass writes Xin^T in bf16, which dW1 reads in the backward)
    HSTU_TRY(hstu::launch_to_bf16_t(XIN, d, T, d, XINT, ts.tp, s, XIN16, 3 * d, true), "bf16 split");
    HSTU_TRY(hstu::launch_to_bf16x3(W1, d4, d, W1_16, 1, s), "bf16 split");
    hstu::GemmBf16Args g{XIN16, 3 * d, W1_16, 3 * d, Z, d4, nullptr, T, d4, 3 * d, 1};
    g.bias = params->b1;
    g.act[0] = U; g.act[1] = V; g.act[2] = Q; g.act[3] = K;
    g.act_w = d;
    if (bf16_bwd) {
      // the bf16 copies of V, Q, K the bf16 attention reads
      g.act16[1] = V16; g.act16[2] = Q16; g.act16[3] = K16;
    }
    HSTU_TRY(hstu::launch_gemm_bf16_f32(g, s), "projection (bf16)");
  } else if (fwd) {
    hstu::GemmF32Args g{};
    g.A = XIN; g.sam = d; g.sak = 1;
    g.B = W1; g.sbk = 1; g.sbn = d;
    g.C = Z; g.ldc = d4; g.bias = params->b1;
    g.outs[0] = U; g.outs[1] = V; g.outs[2] = Q; g.outs[3] = K;
    g.split = d; g.M = static_cast<int>(T); g.N = d4; g.K = d;
    const hipError_t e = hstu::launch_gemm_f32_mma(g, 2, 1, s);
    if (e == hipErrorNotSupported) {
      st = do_proj(desc, params, T, XIN, U, V, Q, K, s);
      if (st) return st;
      HSTU_TRY(hstu::launch_gemm_f32s(XIN, d, 1, W1, 1, d, Z, d4, nullptr, params->b1, static_cast<int>(T), d4,
                                      d, 1, s), "z gemm");
    } else {
      HSTU_TRY(e, "projection");
    }
  }
  if (fwd) {
    if (bf16_bwd && !g16) {
      // the bf16 copies of Q, K, V that the attention reads (kept in the
      // workspace for the two-call step; with g16 the projection wrote them)
      const int64_t n = T * d;
      HSTU_TRY(hstu::launch_to_bf16(Q, Q16, n, s), "bf16 copy");
      HSTU_TRY(hstu::launch_to_bf16(K, K16, n, s), "bf16 copy");
      HSTU_TRY(hstu::launch_to_bf16(V, V16, n, s), "bf16 copy");
    }
    if (fwd16) {
      // AV = (SiLU(a Q K^T + rab) . M) V on the bf16 kernel, fp32 out
      hstu_layer_desc d16 = *desc;
      d16.dtype = HSTU_BF16;
      const hstu::AttnArgs a = make_attn_args(&d16, jagged, nullptr, Q16, K16, V16, params->pos_bias,
                                              params->time_bias, AV, attn16_ws);
      HSTU_TRY(hstu::launch_attn_bf16(a, s), "attention forward (bf16)");
    } else if (bf16_bwd) {
      // head_dim 32: the row-structured bf16 kernel, from the same copies
      hstu::BwdAttnArgs fa = ba;
      fa.q16 = Q16; fa.k16 = K16; fa.v16 = V16;
      HSTU_TRY(hstu::launch_attn_fwd_bf16_rows(fa, s), "attention forward (bf16)");
    } else {
      HSTU_TRY(hstu::launch_attn_train_fwd(ba, s), "attention forward");
    }
    // (with the bf16 products G goes out in bf16 only: f2 and dW2 read it so)
    HSTU_TRY(hstu::launch_ln_gate_fwd(AV, U, params->ln_gamma, params->ln_beta, NH, RSTD, g16 ? nullptr : G,
                                      g16 ? G16 : nullptr, T, d, desc->ln_eps, s), "ln/gate forward");
  }
  if (!bwd) {
    // Y = X + G W2^T + b2
    if (g16) {
      HSTU_TRY(hstu::launch_to_bf16(W2, W2_16, static_cast<int64_t>(d) * d, s), "bf16 copy");
      hstu::GemmBf16Args g{G16, d, W2_16, d, static_cast<float*>(y), d, X, T, d, d, 1};
      g.bias = params->b2;
      HSTU_TRY(hstu::launch_gemm_bf16_f32(g, s), "output gemm (bf16)");
    } else {
      HSTU_TRY(hstu::launch_gemm_f32s(G, d, 1, W2, 1, d, static_cast<float*>(y), d, X,
                                      static_cast<const float*>(params->b2), static_cast<int>(T), d, d, 1, s),
               "output gemm");
    }
    return ok();
  }
  // Y = X + G W2^T + b2
  if (g16) {
    // dG = dY W2 (B = W2^T); dW2 = dY^T G over the tokens, in splits
    HSTU_TRY(hstu::launch_to_bf16_t(W2, d, d, d, W2T, d, s), "bf16 transpose");
    // dY^T, the row-major dY copy and db2 (dY's column sums) in one pass over dY
    HSTU_TRY(hstu::launch_to_bf16_t(DY, d, T, d, DYT, ts.tp, s, DY16, d, false, grads->db2), "bf16 transpose");
    HSTU_TRY(hstu::launch_bf16_t(G16, d, T, d, GT, ts.tp, s), "bf16 transpose");
    HSTU_TRY(gemm16(DY16, d, W2T, d, DG, d, nullptr, T, d, d, 1), "dG gemm (bf16)");
    HSTU_TRY(gemm16(DYT, ts.tp, GT, ts.tp, PART, d, nullptr, d, d, ts.kc, ts.S), "dW2 gemm (bf16)");
    HSTU_TRY(hstu::launch_sum_splits(PART, ts.S, static_cast<int64_t>(d) * d, grads->dw2, s), "dW2 sum");
  } else {
    HSTU_TRY(hstu::launch_gemm_f32s(DY, d, 1, W2, d, 1, DG, d, nullptr, nullptr, static_cast<int>(T), d, d, 1,
                                    s), "dG gemm");
    HSTU_TRY(hstu::launch_gemm_f32s(DY, 1, d, G, d, 1, grads->dw2, d, nullptr, nullptr, d, d, T,
                                    splits(d, d), s), "dW2 gemm");
  }
  if (!g16) HSTU_TRY(hstu::launch_colsum(DY, d, T, d, grads->db2, s), "db2");
  // G = (N^ gamma + beta) . U
  // (with the bf16 attention backward, dAV goes out in bf16 only: its one reader)
  HSTU_TRY(hstu::launch_ln_gate_bwd(DG, U, NH, RSTD, params->ln_gamma, params->ln_beta, DZ, d4,
                                    bf16_bwd ? nullptr : DAV, bf16_bwd ? DAV16 : nullptr, grads->dgamma,
                                    grads->dbeta, T, d, s), "ln/gate backward");
  // AV = (SiLU(a Q K^T + rab) . M) V, per head
  ba.dav = bf16_bwd ? nullptr : DAV;
  ba.dv = DZ + d; ba.dq = DZ + 2 * d; ba.dk = DZ + 3 * d; ba.ld_dz = d4;
  ba.dpos = grads->dpos; ba.dtime = grads->dtime;
  if (bf16_bwd) {
    ba.q16 = Q16; ba.k16 = K16; ba.v16 = V16; ba.dav16 = DAV16;
    HSTU_TRY(hstu::launch_attn_bwd_bf16(ba, s), "attention backward (bf16)");
  } else {
    HSTU_TRY(hstu::launch_attn_bwd_f32(ba, s), "attention backward");
  }
  // [U V Q K] = SiLU(X W1^T + b1)
  if (g16) {
    // dZ in bf16 (row-major and transposed) and db1 in one pass; dW1 = dZ^T
    // Xin over the tokens, in splits; dX (or dXn) = dZ W1 (B = W1^T)
    HSTU_TRY(hstu::launch_silu_bwd_bf16(DZ, Z, T, d4, DZ16, DZT, ts.tp, grads->db1, s), "silu backward (bf16)");
    HSTU_TRY(hstu::launch_to_bf16_t(W1, d, d4, d, W1T, d4, s), "bf16 transpose");
    HSTU_TRY(gemm16(DZT, ts.tp, XINT, ts.tp, PART, d, nullptr, d4, d, ts.kc, ts.S), "dW1 gemm (bf16)");
    HSTU_TRY(hstu::launch_sum_splits(PART, ts.S, static_cast<int64_t>(d4) * d, grads->dw1, s), "dW1 sum");
    if (norm1) {
      HSTU_TRY(gemm16(DZ16, d4, W1T, d4, DG, d, nullptr, T, d, d4, 1), "dXn gemm (bf16)");
      HSTU_TRY(hstu::launch_ln1_bwd(X, DG, DY, params->ln1_gamma, static_cast<float*>(dx), grads->dln1_gamma,
                                    grads->dln1_beta, T, d, desc->ln_eps, s), "input LayerNorm backward");
    } else {
      HSTU_TRY(gemm16(DZ16, d4, W1T, d4, static_cast<float*>(dx), d, DY, T, d, d4, 1), "dX gemm (bf16)");
    }
    return ok();
  }
  HSTU_TRY(hstu::launch_silu_bwd(DZ, Z, T * d4, s), "silu backward");
  HSTU_TRY(hstu::launch_colsum(DZ, d4, T, d4, grads->db1, s), "db1");
  HSTU_TRY(hstu::launch_gemm_f32s(DZ, 1, d4, XIN, d, 1, grads->dw1, d, nullptr, nullptr, d4, d, T,
                                  splits(d4, d), s), "dW1 gemm");
  if (norm1) {
    // d LayerNorm(X) = dZ W1 (into DG, free by now), then back through the LayerNorm, plus dY
    HSTU_TRY(hstu::launch_gemm_f32s(DZ, d4, 1, W1, d, 1, DG, d, nullptr, nullptr, static_cast<int>(T), d, d4, 1,
                                    s), "dXn gemm");
    HSTU_TRY(hstu::launch_ln1_bwd(X, DG, DY, params->ln1_gamma, static_cast<float*>(dx), grads->dln1_gamma,
                                  grads->dln1_beta, T, d, desc->ln_eps, s), "input LayerNorm backward");
  } else {
    HSTU_TRY(hstu::launch_gemm_f32s(DZ, d4, 1, W1, d, 1, static_cast<float*>(dx), d, DY, nullptr,
                                    static_cast<int>(T), d, d4, 1, s), "dX gemm");
  }
#undef HSTU_TRY
  return ok();
}

}  // namespace

int hstu_layer_bwd(const hstu_layer_desc* desc, const hstu_layer_params* params,
                   const hstu_jagged* jagged, const void* x, const void* dy, void* dx,
                   const hstu_layer_grads* grads, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return layer_train(desc, params, jagged, x, dy, dx, nullptr, grads, workspace, workspace_bytes, stream,
                     kTrainFull);
}

int hstu_layer_fwd_train(const hstu_layer_desc* desc, const hstu_layer_params* params,
                         const hstu_jagged* jagged, const void* x, void* y, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return layer_train(desc, params, jagged, x, nullptr, nullptr, y, nullptr, workspace, workspace_bytes,
                     stream, kTrainForward);
}

int hstu_layer_bwd_after_fwd(const hstu_layer_desc* desc, const hstu_layer_params* params,
                             const hstu_jagged* jagged, const void* x, const void* dy, void* dx,
                             const hstu_layer_grads* grads, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return layer_train(desc, params, jagged, x, dy, dx, nullptr, grads, workspace, workspace_bytes, stream,
                     kTrainBackward);
}

int hstu_embed_fwd(int64_t T, int32_t d_model, int32_t dtype, const void* item_emb,
                   int64_t num_items, const void* action_emb, int32_t num_actions,
                   const int64_t* item_ids, const int32_t* actions, void* x, void* stream) {
  CHECK(dtype == HSTU_F32 || dtype == HSTU_BF16, HSTU_E_INVAL, "unknown dtype %d", dtype);
  CHECK(T >= 0 && d_model > 0 && num_items >= 0 && num_actions >= 0, HSTU_E_INVAL, "bad sizes");
  CHECK(d_model % 8 == 0, HSTU_E_UNSUPPORTED, "d_model must be a multiple of 8");
  if (T == 0) return ok();
  CHECK(item_emb && action_emb && item_ids && actions && x, HSTU_E_INVAL, "NULL pointer");
  CHECK(aligned16(item_emb) && aligned16(action_emb) && aligned16(x), HSTU_E_INVAL,
        "tables and x must be 16-byte aligned");
  hstu::EmbedArgs a{item_emb, action_emb, item_ids, actions, x, T, num_items, num_actions, d_model};
  return device_status(dtype == HSTU_BF16 ? hstu::launch_embed_bf16(a, as_stream(stream))
                                          : hstu::launch_embed_f32(a, as_stream(stream)),
                       "embed launch");
}

int hstu_check_inputs(const hstu_layer_desc* desc, const hstu_jagged* jagged,
                      const hstu_kv_cache* cache, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  st = check_jagged(desc, jagged, cache);
  if (st) return st;
  const int B = jagged->num_seqs;
  hipStream_t s = as_stream(stream);
  std::vector<int64_t> off(B + 1, 0), coff;
  std::vector<int32_t> tgt;
  hipError_t e = hipSuccess;
  if (B > 0) e = hipMemcpyAsync(off.data(), jagged->offsets, sizeof(int64_t) * (B + 1),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && B > 0 && jagged->num_targets) {
    tgt.resize(B);
    e = hipMemcpyAsync(tgt.data(), jagged->num_targets, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess && B > 0 && cache) {
    coff.resize(B + 1);
    e = hipMemcpyAsync(coff.data(), cache->offsets, sizeof(int64_t) * (B + 1), hipMemcpyDeviceToHost, s);
  }
  std::vector<int32_t> ty, cty;
  if (e == hipSuccess && typed(desc) && jagged->total_tokens > 0) {
    ty.resize(static_cast<size_t>(jagged->total_tokens));
    e = hipMemcpyAsync(ty.data(), jagged->token_types, sizeof(int32_t) * ty.size(), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess && typed(desc) && cache && cache->total_tokens > 0) {
    cty.resize(static_cast<size_t>(cache->total_tokens));
    e = hipMemcpyAsync(cty.data(), cache->token_types, sizeof(int32_t) * cty.size(), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_status(e, "check_inputs copy");
  CHECK(B == 0 || off[0] == 0, HSTU_E_DATA, "offsets[0] = %lld, expected 0", static_cast<long long>(off[0]));
  for (int b = 0; b < B; ++b) {
    const int64_t L = off[b + 1] - off[b];
    CHECK(L >= 0, HSTU_E_DATA, "offsets decrease at sequence %d", b);
    CHECK(L <= jagged->max_seq_len, HSTU_E_DATA, "sequence %d has length %lld > max_seq_len %d", b,
          static_cast<long long>(L), jagged->max_seq_len);
    if (!tgt.empty())
      CHECK(tgt[b] >= 0 && tgt[b] <= L, HSTU_E_DATA, "num_targets[%d] = %d outside [0, %lld]", b, tgt[b],
            static_cast<long long>(L));
    int64_t C = 0;
    if (cache) {
      C = coff[b + 1] - coff[b];
      CHECK(C >= 0 && C <= cache->max_len, HSTU_E_DATA, "cache length of sequence %d is %lld (max_len %d)",
            b, static_cast<long long>(C), cache->max_len);
    }
    // largest visible position difference: the last query against cache row 0
    // (or own token 0); targets sit at C + (L - m)
    const int64_t m = tgt.empty() ? 0 : tgt[b];
    const int64_t max_dp = L == 0 ? 0 : (m > 0 ? C + (L - m) : C + L - 1);
    const int64_t n_max = (static_cast<int64_t>(desc->pos_table_len) + 1) / 2;
    CHECK(linear_bias(desc) || max_dp <= n_max - 1, HSTU_E_DATA,
          "sequence %d needs position differences up to %lld but the table covers %lld", b,
          static_cast<long long>(max_dp), static_cast<long long>(n_max - 1));
  }
  CHECK(B == 0 || off[B] == jagged->total_tokens, HSTU_E_DATA, "offsets[B] = %lld != total_tokens %lld",
        static_cast<long long>(B ? off[B] : 0), static_cast<long long>(jagged->total_tokens));
  if (cache && B > 0) {
    CHECK(coff[0] == 0 && coff[B] == cache->total_tokens, HSTU_E_DATA,
          "cache offsets must start at 0 and end at cache total_tokens");
  }
  for (size_t i = 0; i < ty.size(); ++i)
    CHECK(ty[i] >= 0 && ty[i] < desc->num_token_types, HSTU_E_DATA, "token_types[%zu] = %d outside [0, %d)", i,
          ty[i], desc->num_token_types);
  for (size_t i = 0; i < cty.size(); ++i)
    CHECK(cty[i] >= 0 && cty[i] < desc->num_token_types, HSTU_E_DATA,
          "cache token_types[%zu] = %d outside [0, %d)", i, cty[i], desc->num_token_types);
  return ok();
}

}  // extern "C"
