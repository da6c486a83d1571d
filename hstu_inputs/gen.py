"""Seeded synthetic workloads for the HSTU jagged layer forward.

Five workloads are defined, numbered 0..4 (``CONFIG_NAMES``):

0. one fp32 layer, one sequence of 64 tokens, d_model 64, 2 heads of 32;
1. one bf16 layer, 64 sequences with lengths uniform on [16, 512],
   d_model 256, 4 heads of 64;
2. one bf16 layer, 16 sequences with lengths uniform on [2048, 8192] (the
   first fixed at 8192), d_model 512, 8 heads of 64;
3. an 8-layer bf16 stack over 128 sequences with Zipf(1.2) lengths clipped
   to [32, 4096]; tokens are item_emb[x] + action_emb[a] from a 1M x 512 item
   table and a 16 x 512 action table;
4. ranking inference: 32 users, 4096 history tokens each plus 512 candidates
   scored in micro-batches of 128 over a cached history, 4 bf16 layers.

Recipe shared by all workloads (the pages publish no dataset; these stand in
for the public and industrial logs they evaluate on):

* X ~ N(0, 1); f1 weight [4d, d] and f2 weight [d, d] Xavier-uniform with
  bound sqrt(6 / (fan_in + fan_out)); linear biases 0, LayerNorm gamma 1 and
  beta 0 (``affine="random"`` draws non-trivial ones for tests instead);
* timestamps are int64 seconds: the first token of every sequence is at
  1_600_000_000 and each gap is ceil(Exp(mean 300 s)), so they strictly
  increase;
* the position-bias table has 2*N-1 entries (N = the workload's longest
  sequence, history plus candidate for workload 4) and the time-bias table
  has 32 entries; both are N(0, 0.02);
* bf16 workloads round X, W1, W2 and the embedding tables to bf16 with
  round-to-nearest-even and keep them as float32 arrays whose values are all
  exactly representable in bf16. Biases, tables, gamma and beta stay fp32.

Random streams: ``SeedSequence(1000 + k).spawn(...)``, one child stream per
array, in the order the arrays are listed in ``_STREAMS``. Nothing here
performs the layer's arithmetic.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

CONFIG_NAMES = {
    0: "fp32 1x64 d64 h2",
    1: "bf16 64 jagged U[16,512] d256 h4",
    2: "bf16 16 jagged U[2048,8192] d512 h8",
    3: "bf16 8-layer stack 128 Zipf[32,4096] d512 h8 + item/action embeddings",
    4: "bf16 ranking 32 users x (4096 history + 512 candidates, b_m=128) d512 h8 4 layers",
}

T0_SECONDS = 1_600_000_000
GAP_MEAN_SECONDS = 300.0
NUM_TIME_BUCKETS = 32
TABLE_STD = 0.02
LN_EPS = 1e-5


# --------------------------------------------------------------------------
# bf16 helpers (data-type conversion only)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are ``x`` rounded to bf16 (RNE)."""
    bits = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).reshape(np.shape(x))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LayerParams:
    w1: np.ndarray         # [4d, d] float32 (nn.Linear layout: out x in)
    b1: np.ndarray         # [4d] float32
    w2: np.ndarray         # [d, d] float32
    b2: np.ndarray         # [d] float32
    gamma: np.ndarray      # [d] float32
    beta: np.ndarray       # [d] float32
    pos_bias: np.ndarray   # [2*n_max-1] float32
    time_bias: np.ndarray  # [num_time_buckets] float32
    # options (off by default): the input LayerNorm before f1, and the
    # parameter-free position/time bias slopes (m_p, m_t) in place of tables
    input_norm: bool = False
    ln1_gamma: Optional[np.ndarray] = None   # [d] float32
    ln1_beta: Optional[np.ndarray] = None    # [d] float32
    linear_bias: Optional[tuple] = None


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": X, W1, W2 (and embedding tables)
    d_model: int
    num_heads: int
    head_dim: int
    n_max: int                 # position table has 2*n_max-1 entries
    num_time_buckets: int
    alpha: float
    ln_eps: float
    offsets: np.ndarray        # int64 [B+1]
    timestamps: np.ndarray     # int64 [T]
    x: Optional[np.ndarray]    # float32 [T, d]; None when built from embeddings
    layers: List[LayerParams]
    # workload 3 (action-oriented tokens)
    item_emb: Optional[np.ndarray] = None    # float32 [num_items, d]
    action_emb: Optional[np.ndarray] = None  # float32 [num_actions, d]
    item_ids: Optional[np.ndarray] = None    # int64 [T]
    actions: Optional[np.ndarray] = None     # int32 [T]
    # workload 4 (candidates scored against a cached history)
    cand_offsets: Optional[np.ndarray] = None     # int64 [B+1], per-user candidates
    cand_timestamps: Optional[np.ndarray] = None  # int64 [sum m]
    cand_x: Optional[np.ndarray] = None           # float32 [sum m, d]
    micro_batch: Optional[int] = None

    @property
    def num_seqs(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)

    @property
    def max_seq_len(self) -> int:
        return int(self.lengths.max()) if self.num_seqs else 0


# --------------------------------------------------------------------------
# primitive draws
# --------------------------------------------------------------------------

def make_jagged(lengths: Sequence[int]) -> np.ndarray:
    """offsets[B+1] (int64) for the given per-sequence lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    offsets = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    return offsets


def make_timestamps(rng: np.random.Generator, offsets: np.ndarray,
                    t0: int = T0_SECONDS) -> np.ndarray:
    """Per sequence: t_0 = t0 and t_{i+1} = t_i + ceil(Exp(mean 300 s))."""
    total = int(offsets[-1])
    gaps = np.ceil(rng.exponential(GAP_MEAN_SECONDS, size=total)).astype(np.int64)
    gaps = np.maximum(gaps, 1)
    ts = np.empty(total, dtype=np.int64)
    for b in range(offsets.shape[0] - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        if e > s:
            g = gaps[s:e].copy()
            g[0] = 0
            ts[s:e] = t0 + np.cumsum(g)
    return ts


def _xavier(rng: np.random.Generator, out_f: int, in_f: int) -> np.ndarray:
    a = np.sqrt(6.0 / (in_f + out_f))
    return rng.uniform(-a, a, size=(out_f, in_f)).astype(np.float32)


def _normal(rng: np.random.Generator, shape, std=1.0) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def make_layer_params(streams: Dict[str, np.random.Generator], d: int, n_max: int,
                      dtype: str, affine: str = "default",
                      num_time_buckets: int = NUM_TIME_BUCKETS) -> LayerParams:
    """One layer's parameters. Streams used (in order): w1, w2, pos, time and,
    for ``affine="random"``, b1, b2, gamma, beta."""
    w1 = _xavier(streams["w1"], 4 * d, d)
    w2 = _xavier(streams["w2"], d, d)
    if dtype == "bf16":
        w1 = bf16_round(w1)
        w2 = bf16_round(w2)
    pos = _normal(streams["pos"], (2 * n_max - 1,), TABLE_STD)
    tim = _normal(streams["time"], (num_time_buckets,), TABLE_STD)
    if affine == "random":
        b1 = _normal(streams["b1"], (4 * d,), 0.1)
        b2 = _normal(streams["b2"], (d,), 0.1)
        gamma = (1.0 + _normal(streams["gamma"], (d,), 0.1)).astype(np.float32)
        beta = _normal(streams["beta"], (d,), 0.1)
    else:
        b1 = np.zeros(4 * d, np.float32)
        b2 = np.zeros(d, np.float32)
        gamma = np.ones(d, np.float32)
        beta = np.zeros(d, np.float32)
    return LayerParams(w1, b1, w2, b2, gamma, beta, pos, tim)


_LAYER_STREAMS = ("w1", "w2", "pos", "time", "b1", "b2", "gamma", "beta")


def _spawn(seed: int, names: Sequence[str]) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(names))
    return {n: np.random.default_rng(c) for n, c in zip(names, children)}


def _layer_stream_names(num_layers: int) -> List[str]:
    return [f"L{l}.{n}" for l in range(num_layers) for n in _LAYER_STREAMS]


def _layer_streams(all_streams, l):
    return {n: all_streams[f"L{l}.{n}"] for n in _LAYER_STREAMS}


# --------------------------------------------------------------------------
# generic builder (tests use it for shrunken and edge-case workloads)
# --------------------------------------------------------------------------

_STREAMS = ("lengths", "x", "timestamps", "ids", "actions", "item_emb",
            "action_emb", "cand_x", "cand_gap")


def make_custom(lengths: Sequence[int], d_model: int, num_heads: int,
                dtype: str = "bf16", seed: int = 0, num_layers: int = 1,
                n_max: Optional[int] = None, affine: str = "default",
                alpha: float = 1.0, name: str = "custom",
                x_std: float = 1.0) -> Workload:
    """A single- or multi-layer workload over explicit sequence lengths."""
    streams = _spawn(seed, list(_STREAMS) + _layer_stream_names(num_layers))
    offsets = make_jagged(lengths)
    total = int(offsets[-1])
    maxlen = int(np.max(lengths)) if len(lengths) else 1
    n_max = int(n_max if n_max is not None else max(maxlen, 1))
    x = _normal(streams["x"], (total, d_model), x_std)
    if dtype == "bf16":
        x = bf16_round(x)
    ts = make_timestamps(streams["timestamps"], offsets)
    layers = [make_layer_params(_layer_streams(streams, l), d_model, n_max, dtype, affine)
              for l in range(num_layers)]
    return Workload(name=name, dtype=dtype, d_model=d_model, num_heads=num_heads,
                    head_dim=d_model // num_heads, n_max=n_max,
                    num_time_buckets=NUM_TIME_BUCKETS, alpha=alpha, ln_eps=LN_EPS,
                    offsets=offsets, timestamps=ts, x=x, layers=layers)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def _zipf_lengths(rng, n, a, lo, hi):
    return np.clip(rng.zipf(a, size=n), lo, hi).astype(np.int64)


def _zipf_ids(rng, n, a, num_items):
    """Item id = rank - 1 with P(rank = k) proportional to k^-a on 1..num_items
    (inverse CDF over the full table)."""
    ranks = np.arange(1, num_items + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-a))
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), num_items - 1).astype(np.int64)


def make_config(k: int, affine: str = "default", num_items: int = 1_000_000) -> Workload:
    """Workload ``k`` (0..4) drawn from SeedSequence(1000 + k)."""
    seed = 1000 + k
    if k == 0:
        w = make_custom([64], 64, 2, dtype="f32", seed=seed, n_max=64, affine=affine,
                        name=CONFIG_NAMES[0])
        return w
    if k == 1:
        rng = _spawn(seed, ["lengths"])["lengths"]
        lengths = rng.integers(16, 512, size=64, endpoint=True)
        return make_custom(lengths, 256, 4, dtype="bf16", seed=seed + 100_000, n_max=512,
                           affine=affine, name=CONFIG_NAMES[1])
    if k == 2:
        rng = _spawn(seed, ["lengths"])["lengths"]
        lengths = rng.integers(2048, 8192, size=16, endpoint=True)
        lengths[0] = 8192
        return make_custom(lengths, 512, 8, dtype="bf16", seed=seed + 100_000, n_max=8192,
                           affine=affine, name=CONFIG_NAMES[2])
    if k == 3:
        d, layers = 512, 8
        streams = _spawn(seed, list(_STREAMS) + _layer_stream_names(layers))
        lengths = _zipf_lengths(streams["lengths"], 128, 1.2, 32, 4096)
        offsets = make_jagged(lengths)
        total = int(offsets[-1])
        ts = make_timestamps(streams["timestamps"], offsets)
        item_emb = bf16_round(_normal(streams["item_emb"], (num_items, d), TABLE_STD))
        action_emb = bf16_round(_normal(streams["action_emb"], (16, d), TABLE_STD))
        ids = _zipf_ids(streams["ids"], total, 1.1, num_items)
        acts = streams["actions"].integers(0, 16, size=total).astype(np.int32)
        params = [make_layer_params(_layer_streams(streams, l), d, 4096, "bf16", affine)
                  for l in range(layers)]
        return Workload(name=CONFIG_NAMES[3], dtype="bf16", d_model=d, num_heads=8,
                        head_dim=64, n_max=4096, num_time_buckets=NUM_TIME_BUCKETS,
                        alpha=1.0, ln_eps=LN_EPS, offsets=offsets, timestamps=ts, x=None,
                        layers=params, item_emb=item_emb, action_emb=action_emb,
                        item_ids=ids, actions=acts)
    if k == 4:
        return make_ranking(seed=seed, users=32, history=4096, candidates=512,
                            micro_batch=128, d_model=512, num_heads=8, num_layers=4,
                            affine=affine, name=CONFIG_NAMES[4])
    raise ValueError(f"unknown workload {k}")


def make_ranking(seed: int, users: int, history, candidates, micro_batch: int,
                 d_model: int, num_heads: int, num_layers: int, affine: str = "default",
                 name: str = "ranking", dtype: str = "bf16") -> Workload:
    """History sequences plus per-user candidates. ``history`` and
    ``candidates`` are ints (same for every user) or per-user sequences.
    All candidates of a user share one request timestamp
    t_req = t_last + ceil(Exp(300 s))."""
    streams = _spawn(seed, list(_STREAMS) + _layer_stream_names(num_layers))
    hist = np.broadcast_to(np.asarray(history, np.int64), (users,)).copy()
    cand = np.broadcast_to(np.asarray(candidates, np.int64), (users,)).copy()
    offsets = make_jagged(hist)
    cand_offsets = make_jagged(cand)
    n_max = int((hist + 1).max())  # candidates sit at position n (one past history)
    x = _normal(streams["x"], (int(offsets[-1]), d_model))
    cx = _normal(streams["cand_x"], (int(cand_offsets[-1]), d_model))
    if dtype == "bf16":
        x, cx = bf16_round(x), bf16_round(cx)
    ts = make_timestamps(streams["timestamps"], offsets)
    gap = np.maximum(np.ceil(streams["cand_gap"].exponential(GAP_MEAN_SECONDS, size=users)), 1)
    cts = np.empty(int(cand_offsets[-1]), np.int64)
    for u in range(users):
        last = ts[offsets[u + 1] - 1] if hist[u] > 0 else T0_SECONDS
        cts[cand_offsets[u]:cand_offsets[u + 1]] = int(last) + int(gap[u])
    params = [make_layer_params(_layer_streams(streams, l), d_model, n_max, dtype, affine)
              for l in range(num_layers)]
    return Workload(name=name, dtype=dtype, d_model=d_model, num_heads=num_heads,
                    head_dim=d_model // num_heads, n_max=n_max,
                    num_time_buckets=NUM_TIME_BUCKETS, alpha=1.0, ln_eps=LN_EPS,
                    offsets=offsets, timestamps=ts, x=x, layers=params,
                    cand_offsets=cand_offsets, cand_timestamps=cts, cand_x=cx,
                    micro_batch=micro_batch)


def micro_batches(w: Workload, b_m: Optional[int] = None):
    """Split every user's candidates into consecutive micro-batches of b_m.

    Yields (offsets, row_index) per micro-batch: ``offsets`` is the jagged
    layout of the micro-batch (one sequence per user, possibly empty) and
    ``row_index`` are the rows of ``cand_x`` it holds, user-major."""
    b_m = int(b_m or w.micro_batch)
    cl = np.diff(w.cand_offsets)
    nmb = int(np.max((cl + b_m - 1) // b_m)) if cl.size else 0
    for mb in range(nmb):
        lens, rows = [], []
        for u in range(cl.shape[0]):
            s = int(w.cand_offsets[u]) + mb * b_m
            e = min(int(w.cand_offsets[u + 1]), s + b_m)
            n = max(0, e - s)
            lens.append(n)
            rows.append(np.arange(s, s + n, dtype=np.int64))
        yield make_jagged(lens), np.concatenate(rows) if rows else np.zeros(0, np.int64)
