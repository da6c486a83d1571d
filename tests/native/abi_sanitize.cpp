// Host-only driver for the C ABI's validation, sizing and host sampler,
// built with AddressSanitizer and UndefinedBehaviorSanitizer together with
// the library's host sources (api.cpp, plan.cpp, sampler.cpp). The device
// launchers are replaced by stubs that abort: every call made here must be
// answered on the host, so no GPU is needed. Run by tests/test_sanitizers.py.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "hstu.h"

namespace {

int failures = 0;

#define EXPECT(cond)                                                                \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "%s:%d: expected %s (last error: %s)\n", __FILE__,       \
                   __LINE__, #cond, hstu_last_error());                             \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

// never dereferenced: validation rejects or returns before any launch
void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t{0x100000} + off); }

hstu_layer_desc desc(int d = 512, int H = 8, int dtype = HSTU_BF16, int pos = 255) {
  hstu_layer_desc x;
  std::memset(&x, 0, sizeof(x));
  x.d_model = d;
  x.num_heads = H;
  x.head_dim = d / H;
  x.dtype = dtype;
  x.alpha = 1.0f;
  x.ln_eps = 1e-5f;
  x.pos_table_len = pos;
  x.num_time_buckets = 32;
  return x;
}

hstu_jagged jag(int B = 2, int64_t T = 10, int mx = 6) {
  hstu_jagged j;
  std::memset(&j, 0, sizeof(j));
  j.num_seqs = B;
  j.max_seq_len = mx;
  j.total_tokens = T;
  j.offsets = static_cast<const int64_t*>(fake());
  j.timestamps = static_cast<const int64_t*>(fake());
  return j;
}

int attn(const hstu_layer_desc* d, const hstu_jagged* j, const hstu_kv_cache* c = nullptr,
         uintptr_t p = 0x100000, size_t ws = size_t{1} << 20) {
  void* q = reinterpret_cast<void*>(p);
  return hstu_attn_fwd(d, j, c, q, q, q, static_cast<const float*>(q), static_cast<const float*>(q),
                       static_cast<float*>(q), fake(), ws, nullptr);
}

void attention_validation() {
  EXPECT(attn(nullptr, nullptr) == HSTU_E_INVAL);
  hstu_jagged j = jag();
  EXPECT(attn(nullptr, &j) == HSTU_E_INVAL);
  hstu_layer_desc d = desc();
  d.head_dim = 32;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc(256, 16);   // head_dim 16
  EXPECT(attn(&d, &j) == HSTU_E_UNSUPPORTED);
  for (float a : {0.0f, NAN, 1e9f, -INFINITY}) {
    d = desc();
    d.alpha = a;
    EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  }
  d = desc(512, 8, HSTU_BF16, 256);
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc(512, 8, HSTU_BF16, 9);
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  d.num_time_buckets = 0;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  d.num_time_buckets = 65;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  d.dtype = 7;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  hstu_kv_cache c;
  std::memset(&c, 0, sizeof(c));
  c.offsets = static_cast<const int64_t*>(fake());
  c.timestamps = static_cast<const int64_t*>(fake());
  c.k = c.v = fake();
  c.max_len = 125;
  c.total_tokens = 100;
  EXPECT(attn(&d, &j, &c) == HSTU_E_INVAL);
  hstu_jagged bad = jag(-1);
  EXPECT(attn(&d, &bad) == HSTU_E_INVAL);
  bad = jag(2, -5);
  EXPECT(attn(&d, &bad) == HSTU_E_INVAL);
  bad = jag(2, 10, 1 << 30);
  EXPECT(attn(&d, &bad) != HSTU_OK);
  EXPECT(attn(&d, &j, nullptr, 0x100008) == HSTU_E_INVAL);
  EXPECT(attn(&d, &j, nullptr, 0) == HSTU_E_INVAL);
  // empty batches return before touching anything
  hstu_jagged e = jag(0, 0, 0);
  EXPECT(attn(&d, &e) == HSTU_OK);
  e = jag(3, 0, 0);
  EXPECT(attn(&d, &e) == HSTU_OK);
  // workspace too small
  const size_t need = hstu_attn_workspace_size(&d, &j);
  EXPECT(need > 0);
  EXPECT(attn(&d, &j, nullptr, 0x100000, need - 1) == HSTU_E_WORKSPACE);
  // bias modes and token types
  d = desc();
  d.num_token_types = HSTU_MAX_TOKEN_TYPES + 1;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  d.bias_mode = 5;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  d.bias_mode = HSTU_BIAS_LINEAR;
  d.linear_m_t = NAN;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);
  d = desc();
  d.num_token_types = 3;
  EXPECT(attn(&d, &j) == HSTU_E_INVAL);   // token_types NULL
}

void noalloc_validation() {
  // a work list beyond the static scratch is refused before the scratch is
  // resolved: 100000 sequences of 8192 tokens
  hstu_layer_desc d = desc();
  hstu_jagged j = jag(100000, 200000, 8192);
  d.pos_table_len = 2 * 8192 - 1;
  void* q = fake();
  EXPECT(hstu_attn_fwd_noalloc(&d, &j, nullptr, q, q, q, static_cast<const float*>(q),
                               static_cast<const float*>(q), static_cast<float*>(q), nullptr) ==
         HSTU_E_WORKSPACE);
}

void sizes() {
  // sizing over a range of shapes: no overflow, monotone in the token count
  for (int B : {1, 2, 7, 64, 513, 100000})
    for (int mx : {1, 63, 64, 65, 8192}) {
      hstu_layer_desc d = desc(512, 8, HSTU_BF16, 2 * mx - 1);
      hstu_jagged j1 = jag(B, static_cast<int64_t>(B) * mx, mx);
      hstu_jagged j2 = jag(B, static_cast<int64_t>(B) * mx / 2 + 1, mx);
      EXPECT(hstu_attn_workspace_size(&d, &j1) >= hstu_attn_workspace_size(&d, &j2));
      EXPECT(hstu_layer_workspace_size(&d, &j1) >= hstu_attn_workspace_size(&d, &j1));
      hstu_layer_desc f = desc(64, 2, HSTU_F32, 2 * mx - 1);
      EXPECT(hstu_attn_workspace_size(&f, &j1) == 0);
      (void)hstu_layer_bwd_workspace_size(&f, &j1);
    }
}

void other_entry_points() {
  hstu_layer_desc d = desc();
  hstu_layer_params pp;
  std::memset(&pp, 0, sizeof(pp));
  pp.w1 = pp.w2 = fake();
  EXPECT(hstu_proj_fwd(&d, &pp, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == HSTU_OK);
  EXPECT(hstu_proj_fwd(&d, &pp, -1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_proj_fwd(&d, nullptr, 4, fake(), fake(4096), fake(8192), fake(12288), fake(16384), nullptr) ==
         HSTU_E_INVAL);
  EXPECT(hstu_norm_gate_fwd(&d, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == HSTU_OK);
  EXPECT(hstu_norm_gate_fwd(&d, -1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_out_fwd(&d, 5, fake(), fake(), fake(), nullptr, fake(), nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_layernorm_fwd(&d, 0, nullptr, nullptr, nullptr, nullptr, nullptr) == HSTU_OK);
  EXPECT(hstu_layernorm_fwd(&d, 4, fake(), nullptr, nullptr, fake(), nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_linear_bias_tables(&d, NAN, 0.1f, static_cast<float*>(fake()),
                                 static_cast<float*>(fake(4096)), nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_linear_bias_tables(&d, 0.1f, 0.1f, static_cast<float*>(fake()), static_cast<float*>(fake()),
                                 nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_embed_fwd(0, 512, HSTU_BF16, nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr, nullptr) ==
         HSTU_OK);
  EXPECT(hstu_embed_fwd(4, 12, HSTU_BF16, fake(), 1, fake(), 1, static_cast<const int64_t*>(fake()),
                        static_cast<const int32_t*>(fake()), fake(), nullptr) == HSTU_E_UNSUPPORTED);
  EXPECT(hstu_gather_rows(-1, 8, nullptr, 1, fake(), fake(4096), nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_gather_rows(4, 12, static_cast<const int64_t*>(fake()), 1, fake(), fake(4096), nullptr) ==
         HSTU_E_INVAL);
  EXPECT(hstu_gather_rows(4, 8, static_cast<const int64_t*>(fake()), 1, fake(), fake(), nullptr) ==
         HSTU_E_INVAL);
  // cache concatenation
  hstu_kv_cache a, n;
  std::memset(&a, 0, sizeof(a));
  a.offsets = static_cast<const int64_t*>(fake());
  a.timestamps = static_cast<const int64_t*>(fake());
  a.k = a.v = fake();
  a.max_len = 8;
  a.total_tokens = 10;
  n = a;
  n.offsets = static_cast<const int64_t*>(fake(1024));
  n.timestamps = static_cast<const int64_t*>(fake(2048));
  n.k = fake(4096);
  n.v = fake(8192);
  n.total_tokens = 5;
  auto o = [](uintptr_t x) { return fake(x); };
  EXPECT(hstu_kv_cache_concat(&d, -1, &a, &n, static_cast<int64_t*>(o(65536)), static_cast<int64_t*>(o(131072)),
                              o(262144), o(524288), nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_kv_cache_concat(&d, 2, nullptr, &n, static_cast<int64_t*>(o(65536)),
                              static_cast<int64_t*>(o(131072)), o(262144), o(524288), nullptr) == HSTU_E_INVAL);
  EXPECT(hstu_kv_cache_concat(&d, 2, &a, &n, static_cast<int64_t*>(o(65536)), static_cast<int64_t*>(o(131072)),
                              fake(), o(524288), nullptr) == HSTU_E_INVAL);
  // the backward pass
  hstu_layer_desc f = desc(64, 2, HSTU_F32, 255);
  hstu_layer_params p;
  std::memset(&p, 0, sizeof(p));
  p.w1 = p.w2 = fake();
  p.pos_bias = p.time_bias = static_cast<const float*>(fake());
  hstu_layer_grads g;
  std::memset(&g, 0, sizeof(g));
  hstu_jagged j = jag();
  const size_t ws = hstu_layer_bwd_workspace_size(&f, &j);
  EXPECT(hstu_layer_bwd(&f, &p, &j, fake(), fake(8192), fake(4096), &g, fake(), ws, nullptr) == HSTU_E_INVAL);
  hstu_layer_desc b = desc();
  EXPECT(hstu_layer_bwd(&b, &p, &j, fake(), fake(8192), fake(4096), &g, fake(), ws, nullptr) ==
         HSTU_E_UNSUPPORTED);
  // the layer
  const size_t lws = hstu_layer_workspace_size(&d, &j);
  EXPECT(hstu_layer_fwd(&d, &p, &j, nullptr, fake(), fake(4096), nullptr, nullptr, fake(), lws - 1, nullptr) ==
         HSTU_E_WORKSPACE);
  EXPECT(hstu_layer_fwd(&d, &p, &j, nullptr, fake(), fake(), nullptr, nullptr, fake(), lws, nullptr) ==
         HSTU_E_INVAL);
  EXPECT(hstu_layer_fwd(&d, &p, &j, nullptr, fake(), fake(4096), nullptr, nullptr, fake(16), lws, nullptr) ==
         HSTU_E_INVAL);
}

// The host sampler over random batches (lengths, alpha, n_max, draws):
// kept rows are increasing within each sequence, within the sequence's own
// range, and the truncated length is floor(n_max^(alpha/2)).
void sampler() {
  std::mt19937_64 rng(1234);
  for (int trial = 0; trial < 300; ++trial) {
    const int B = static_cast<int>(rng() % 40);
    const int64_t n_max = 1 + static_cast<int64_t>(rng() % 600);
    const double alpha = 0.05 + 1.95 * std::uniform_real_distribution<double>(0, 1)(rng);
    std::vector<int64_t> off(B + 1, 0);
    for (int b = 0; b < B; ++b) off[b + 1] = off[b] + static_cast<int64_t>(rng() % 700);
    const int64_t T = off[B];
    std::vector<double> u(B), keys(static_cast<size_t>(T));
    for (auto& x : u) x = std::uniform_real_distribution<double>(0, 1)(rng);
    for (auto& x : keys) x = static_cast<double>(rng() % 50);   // many ties
    std::vector<int64_t> out_off(B + 1), rows(static_cast<size_t>(T) + 1);
    int64_t total = -1;
    const int st = hstu_stochastic_length(B, off.data(), alpha, n_max, u.data(), keys.data(), out_off.data(),
                                          rows.data(), T, &total);
    EXPECT(st == HSTU_OK);
    if (st != HSTU_OK) continue;
    EXPECT(total >= 0 && total <= T && out_off[B] == total);
    const int64_t k = static_cast<int64_t>(std::floor(std::pow(static_cast<double>(n_max), alpha / 2)));
    for (int b = 0; b < B; ++b) {
      const int64_t L = off[b + 1] - off[b], n = out_off[b + 1] - out_off[b];
      EXPECT(n == L || n == k);
      for (int64_t r = out_off[b]; r < out_off[b + 1]; ++r) {
        EXPECT(rows[r] >= off[b] && rows[r] < off[b + 1]);
        if (r > out_off[b]) EXPECT(rows[r] > rows[r - 1]);
      }
    }
    if (T > 0) {
      EXPECT(hstu_stochastic_length(B, off.data(), alpha, n_max, u.data(), keys.data(), out_off.data(),
                                    rows.data(), -1, &total) != HSTU_OK);
    }
  }
  std::vector<int64_t> off = {0, 5, 3};
  std::vector<double> u = {0.5, 0.5}, keys(5, 0.0);
  std::vector<int64_t> oo(3), rows(8);
  int64_t total = 0;
  EXPECT(hstu_stochastic_length(2, off.data(), 1.0, 4, u.data(), keys.data(), oo.data(), rows.data(), 8,
                                &total) == HSTU_E_INVAL);   // decreasing offsets
  off = {0, 5, 9};
  EXPECT(hstu_stochastic_length(2, off.data(), 2.5, 4, u.data(), keys.data(), oo.data(), rows.data(), 8,
                                &total) == HSTU_E_INVAL);   // alpha outside (0, 2]
  EXPECT(hstu_stochastic_length(2, off.data(), 1.0, 0, u.data(), keys.data(), oo.data(), rows.data(), 8,
                                &total) == HSTU_E_INVAL);   // n_max < 1
}

}  // namespace

int main() {
  EXPECT(hstu_abi_version() == HSTU_ABI_VERSION);
  attention_validation();
  noalloc_validation();
  sizes();
  other_entry_points();
  sampler();
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("abi_sanitize: all host checks passed\n");
  return 0;
}
