// Host-side launch planning: the bf16 attention's work items, key-range
// splits and the workspace they need, and the head sizes of the fp32
// training kernels. Plain C++ (no device code), so that
// the C ABI's validation and sizing can also be built on its own for the
// host sanitizer checks.
#include <algorithm>

#include "internal.h"

namespace hstu {

int attn_heads_per_group(int num_heads) {
  for (int c : {8, 4, 2, 1})
    if (num_heads % c == 0) return c;
  return 1;
}

AttnPlan attn_plan(int num_seqs, int max_seq_len, int num_heads, int64_t total_tokens, int d_model,
                   int max_splits) {
  AttnPlan p{};
  p.bm = kAttnBM;
  p.heads_per_group = attn_heads_per_group(num_heads);
  const int64_t n_qt = (static_cast<int64_t>(max_seq_len) + p.bm - 1) / p.bm;
  const int64_t items = static_cast<int64_t>(num_seqs) * n_qt;
  p.splits = (items <= 0 || items >= kAttnSplitMinUnits)
                 ? 1
                 : static_cast<int>(std::min<int64_t>(kAttnMaxSplits, (kAttnSplitMinUnits + items - 1) / items));
  p.splits = std::max(1, std::min(p.splits, max_splits));
  const size_t sched = static_cast<size_t>(kAttnSchedHead + items * p.splits) * sizeof(int);
  p.sched_bytes = (sched + 255) & ~static_cast<size_t>(255);
  const size_t partial =
      p.splits > 1 ? static_cast<size_t>(p.splits) * total_tokens * d_model * sizeof(float) : 0;
  p.workspace_bytes = p.sched_bytes + partial;
  return p;
}

bool attn_can_fuse_norm_gate(int num_seqs, int max_seq_len, int num_heads, int64_t total_tokens,
                             int d_model) {
  // one head group covers each row, and no key-range splits
  const AttnPlan p = attn_plan(num_seqs, max_seq_len, num_heads, total_tokens, d_model);
  return p.heads_per_group == num_heads && num_heads <= 8 && p.splits == 1;
}

bool attn_train_supported(int head_dim) { return head_dim == 32 || head_dim == 64; }

}  // namespace hstu
