// Stochastic Length ("HSTU：Scaling Law 的首次探索" §7.1.5): the sequence
// sampler of the data loader, on the host. A sequence of length n longer than
// N^(alpha/2) is, with probability p = 1 - N^alpha / n^2, replaced by
// k = floor(N^(alpha/2)) of its tokens, kept in their original order; the
// page prints the thresholds as N_{alpha/2} and N_alpha, read as powers.
// The page leaves the choice of the subsequence open; the tokens with the
// smallest caller-drawn keys are kept (ties to the earlier token).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/hstu.h"
#include "internal.h"

extern "C" int hstu_stochastic_length(int32_t num_seqs, const int64_t* offsets, double alpha,
                                      int64_t n_max, const double* u, const double* keys,
                                      int64_t* out_offsets, int64_t* rows, int64_t rows_capacity,
                                      int64_t* out_total) {
  using hstu::api_fail;
  if (num_seqs < 0 || !offsets || !out_offsets || !out_total)
    return api_fail(HSTU_E_INVAL, "num_seqs >= 0 and offsets/out_offsets/out_total are required");
  if (!(alpha > 0.0 && alpha <= 2.0)) return api_fail(HSTU_E_INVAL, "alpha must be in (0, 2]");
  if (n_max < 1) return api_fail(HSTU_E_INVAL, "n_max must be >= 1");
  if (offsets[0] != 0) return api_fail(HSTU_E_INVAL, "offsets[0] must be 0");
  for (int b = 0; b < num_seqs; ++b)
    if (offsets[b + 1] < offsets[b]) return api_fail(HSTU_E_INVAL, "offsets must not decrease");
  const int64_t T = offsets[num_seqs];
  if (T > 0 && (!u || !keys || !rows)) return api_fail(HSTU_E_INVAL, "u, keys and rows are required");
  if (rows_capacity < T) return api_fail(HSTU_E_INVAL, "rows must hold the %lld input rows",
                                         static_cast<long long>(T));
  for (int b = 0; b < num_seqs; ++b)
    if (!(u[b] >= 0.0 && u[b] <= 1.0)) return api_fail(HSTU_E_INVAL, "u must lie in [0, 1]");
  for (int64_t t = 0; t < T; ++t)
    if (!std::isfinite(keys[t])) return api_fail(HSTU_E_INVAL, "keys must be finite");

  const double N = static_cast<double>(n_max);
  const double thresh = std::pow(N, alpha / 2.0);
  const int64_t k = static_cast<int64_t>(std::floor(thresh));
  std::vector<int64_t> idx;
  int64_t w = 0;
  out_offsets[0] = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t s = offsets[b], n = offsets[b + 1] - s;
    bool cut = false;
    if (static_cast<double>(n) > thresh) {
      const double p = 1.0 - std::pow(N, alpha) / (static_cast<double>(n) * static_cast<double>(n));
      cut = u[b] < p;
    }
    if (!cut) {
      for (int64_t j = 0; j < n; ++j) rows[w++] = s + j;
    } else {
      idx.resize(n);
      std::iota(idx.begin(), idx.end(), int64_t{0});
      const double* ks = keys + s;
      auto before = [ks](int64_t a, int64_t c) { return ks[a] < ks[c] || (ks[a] == ks[c] && a < c); };
      std::nth_element(idx.begin(), idx.begin() + k, idx.end(), before);
      std::sort(idx.begin(), idx.begin() + k);
      for (int64_t j = 0; j < k; ++j) rows[w++] = s + idx[j];
    }
    out_offsets[b + 1] = w;
  }
  *out_total = w;
  hstu::api_ok();
  return HSTU_OK;
}
