// Work list of the bf16 attention: the scheduling pass that orders the
// (sequence, 64-query tile, key chunk) work units for attn_bf16_kernel. It
// runs either in its own one-workgroup kernel (csrc/attn.hip) or, for the
// layer forward, as one extra workgroup of the f1 GEMM launch that precedes
// the attention (csrc/gemm.hip), whose operand ring then lends it LDS.
#pragma once

#include "common.h"
#include "internal.h"

namespace hstu {
namespace sched {

constexpr int kNumXcd = 8;          // XCDs of the chip; workgroup id -> XCD id % 8
constexpr int kCostBuckets = 256;   // cost classes of the per-XCD sort (costs of 255 key steps and more share the last)
constexpr int kSchedHead = kAttnSchedHead;
static_assert(kSchedHead == kNumXcd + 1, "work list header: one counter per XCD, then the total");
constexpr int kListInts = kNumXcd * kCostBuckets;   // LDS counters of the counting sort

struct SeqInfo {
  int64_t s;     // first own token row
  int L;         // own length
  int m;         // number of targets (last m own tokens)
  int64_t cs;    // first cache row
  int nc;        // cache length
};

__device__ __forceinline__ SeqInfo seq_info(const AttnArgs& a, int b) {
  SeqInfo si;
  si.s = a.offsets[b];
  si.L = static_cast<int>(a.offsets[b + 1] - si.s);
  int m = a.num_targets ? a.num_targets[b] : 0;
  si.m = m < 0 ? 0 : (m > si.L ? si.L : m);
  if (a.c_offsets) {
    si.cs = a.c_offsets[b];
    si.nc = static_cast<int>(a.c_offsets[b + 1] - si.cs);
  } else {
    si.cs = 0;
    si.nc = 0;
  }
  return si;
}

// Number of key steps (kAttnBN-key tiles visited) of query tile qt of a
// sequence: the cost the schedule sorts by.
__device__ __forceinline__ int tile_steps(const SeqInfo& si, int qt, int bm) {
  const int q0 = qt * bm;
  const int q_hi = min(q0 + bm, si.L);
  const int nkeys = si.nc + q_hi;
  const int n_kt = (nkeys + kAttnBN - 1) / kAttnBN;
  const int first_tgt = si.L - si.m;
  const int skip_a = (si.nc + first_tgt + kAttnBN - 1) / kAttnBN;
  const int skip_b = max((si.nc + q0) / kAttnBN, skip_a);
  return n_kt - (skip_b - skip_a);
}

// Key steps [lo, hi) of chunk c of an item with n steps: chunks of ceil(n / S)
// steps; trailing chunks may be empty.
__device__ __forceinline__ void chunk_range(int n, int S, int c, int& lo, int& hi) {
  const int per = (n + S - 1) / S;
  lo = min(c * per, n);
  hi = min(lo + per, n);
}

// Cost of work unit u = item * S + chunk: its key steps, at least 1 for a
// non-empty item (an empty chunk still writes its zero partial); 0 for an
// empty tile (never scheduled).
__device__ __forceinline__ int unit_cost(const AttnArgs& a, int n_qt, int u) {
  const int S = a.splits;
  const int i = u / S, ch = u - i * S;
  const int b = i / n_qt, t = i - b * n_qt;
  const SeqInfo si = seq_info(a, b);
  // tiles past max_seq_len (a violated contract) are never reached: t < n_qt
  if (t * a.bm >= si.L) return 0;
  int lo, hi;
  chunk_range(tile_steps(si, t, a.bm), S, ch, lo, hi);
  return max(hi - lo, 1);
}

// Exclusive prefix sum over the NT threads of the block (wave scans by
// shuffles, then one pass over the NT / 64 wave totals); *total receives the
// sum. wsum: NT / 64 LDS slots.
template <int NT>
__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* wsum, long long* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long t = __shfl_up(inc, off, 64);
    if (lane >= off) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    long long w = lane < NW ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      const long long t = __shfl_up(w, off, 64);
      if (lane >= off) w += t;
    }
    if (lane < NW) wsum[lane] = w;
  }
  __syncthreads();
  const long long excl = inc - v + (wave ? wsum[wave - 1] : 0);
  *total = wsum[NW - 1];
  __syncthreads();   // wsum may be reused by the next scan
  return excl;
}

// The work list into a.sched, by a block of NT threads: items are the
// non-empty (sequence, 64-query tile) pairs, each cut into a.splits units of
// consecutive key steps; a unit's cost is its number of key steps.
//  1. Units, in (sequence, tile, chunk) order, are cut into kNumXcd
//     contiguous runs of equal total cost; run x goes to XCD x. The
//     workgroups of one XCD then work on one or a few sequences at a time and
//     share their K/V rows in that XCD's L2.
//  2. Within a run, units are counting-sorted by cost, most expensive first,
//     so that the XCD's compute units finish together.
// a.sched[x] (x = 0..8): first list index of XCD x (a.sched[8] = unit count);
// a.sched[9 + k]: unit ((seq * n_qt + tile) * splits + chunk) at list index k.
// cnt: kListInts LDS ints; wsum: NT / 64 LDS slots.
template <int NT>
__device__ __forceinline__ void build(const AttnArgs& a, int n_qt, int* cnt, long long* wsum) {
  static_assert(kListInts % NT == 0, "counters per thread");
  constexpr int kKeep = 8;   // unit costs per thread kept in registers between the passes
  const int tid = threadIdx.x;
  const int items = a.num_seqs * n_qt * a.splits;
  for (int i = tid; i < kListInts; i += NT) cnt[i] = 0;
  // each thread owns a contiguous chunk of units
  const int per = (items + NT - 1) / NT;
  const int i0 = min(tid * per, items), i1 = min(i0 + per, items);
  int cst[kKeep];
  long long sum = 0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    cst[k] = i0 + k < i1 ? unit_cost(a, n_qt, i0 + k) : 0;
    sum += cst[k];
  }
  for (int i = i0 + kKeep; i < i1; ++i) sum += unit_cost(a, n_qt, i);
  long long total_cost;
  const long long run0 = block_exclusive_scan<NT>(sum, wsum, &total_cost);   // also orders cnt's zeroing
  // sort key: XCD-major, cost descending; the unit's XCD is the run holding
  // the midpoint of its cost interval
  auto key_of = [&](long long run, int c) __attribute__((always_inline)) {
    const int x = static_cast<int>(min(static_cast<long long>(kNumXcd - 1),
                                       ((2 * run + c) * kNumXcd) / (2 * total_cost)));
    return x * kCostBuckets + (kCostBuckets - 1 - min(c, kCostBuckets - 1));
  };
  long long run = run0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    if (cst[k] > 0) atomicAdd(&cnt[key_of(run, cst[k])], 1);
    run += cst[k];
  }
  for (int i = i0 + kKeep; i < i1; ++i) {
    const int c = unit_cost(a, n_qt, i);
    if (c > 0) atomicAdd(&cnt[key_of(run, c)], 1);
    run += c;
  }
  __syncthreads();
  // exclusive scan of the counters, kPer per thread
  constexpr int kPer = kListInts / NT;
  int loc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) loc += cnt[tid * kPer + i];
  long long units;
  int base = static_cast<int>(block_exclusive_scan<NT>(loc, wsum, &units));
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = cnt[tid * kPer + i];
    cnt[tid * kPer + i] = base;
    base += c;
  }
  __syncthreads();
  if (tid < kNumXcd) a.sched[tid] = cnt[tid * kCostBuckets];
  if (tid == kNumXcd) a.sched[kNumXcd] = static_cast<int>(units);
  run = run0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    if (cst[k] > 0) a.sched[kSchedHead + atomicAdd(&cnt[key_of(run, cst[k])], 1)] = i0 + k;
    run += cst[k];
  }
  for (int i = i0 + kKeep; i < i1; ++i) {
    const int c = unit_cost(a, n_qt, i);
    if (c > 0) a.sched[kSchedHead + atomicAdd(&cnt[key_of(run, c)], 1)] = i;
    run += c;
  }
}

}  // namespace sched
}  // namespace hstu
