"""Float64 CPU oracle of the HSTU layer forward on jagged sequences.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code, constants or helpers with the HIP library.

Every function is the plain definition, evaluated in float64 with NumPy,
looping over sequences and heads with dense per-sequence matrices. Pages
cited (by title; section, equation or figure):

[GR-7.1]   "HSTU：Scaling Law 的首次探索" (fun-rec mdbook, chapter 7.1)
[NOTES]    "万亿参数推荐大模型：HSTU 架构如何超越传统 Self-Attention"
           (reading notes on arXiv:2402.17152)
[GENRANK]  "6.2. HSTU的工程突破" (fun-rec, chapter 6.2, GenRank)
[SA2HSTU]  "从自注意力到 HSTU：解构下一代推荐系统引擎"

Readings taken where the pages leave a step open:

* score scale alpha defaults to 1: the layer equations in [NOTES] §2.1 and
  [SA2HSTU] step 2 carry no 1/sqrt(d) (only [GENRANK] eq. 6.2.3 restates the
  score with one); alpha is a parameter;
* phi2(.) V(X) is a matrix product ([NOTES] §2.1 and [SA2HSTU] step 2 print
  a product; the element-wise sign in [GR-7.1] §7.1.4 cannot apply to an
  N x N by N x d pair);
* no softmax and no normalisation of the SiLU weights ([GR-7.1] §7.1.4,
  innovation 1);
* the causal mask keeps the diagonal (j <= i);
* the residual Y = X + f2(...) comes from the block diagram of [NOTES] §2.1
  ("残差连接", residual connection); no LayerNorm before f1 by default (the
  layer equations have none); the diagram's Norm1 is an option, and the
  residual then still carries the raw X, since the skip leaves the input
  ahead of Norm1;
* the parameter-free bias of [GENRANK] eq. 6.2.6 is an option of the
  attention (scalars m_p, m_t shared by all heads);
* Norm is LayerNorm over all d features of the token, biased variance,
  eps from the caller (1e-5), affine gamma/beta;
* Split order is U, V, Q, K, contiguous chunks of width d; head h owns
  columns [h*dh, (h+1)*dh) of each chunk;
* rab_{p,t}(i, j) = pos_bias[(p_i - p_j) + n_max - 1]
                  + time_bias[min(nb - 1, floor(log2(|t_i - t_j| + 1)))],
  shared by all heads ([GR-7.1] §7.1.4 innovation 2 names the position and
  time differences; the bucketed time difference follows [GENRANK] eq.
  6.2.6's bucket(t_i - t_j)); the floor(log2) is taken in integers;
* the type-aware term of rab ([GR-7.1] §7.1.4 innovation 2, an option):
  with nt token types, the time table is one table per ordered pair of
  (query type, key type), time_bias[(type_i * nt + type_j) * nb + bucket],
  so each type pair has its own time decay; the position table is shared;
  nt = 1 is the untyped rab;
* targets (ranking candidates, [GR-7.1] §7.1.5 M-FALCON and [GENRANK]
  §6.2.2 Fig. 6.2.2): history is causal, a candidate sees the whole history
  and itself but no other candidate; all candidates of a sequence share the
  "next" position n + (L - m).

Visibility, in one rule: within sequence b the keys are [its cache rows,
then its own tokens]. Key j is visible to query i iff j is a cache row, or
j <= i and (j is not a target or j == i) (own-token indices).
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# scalar pieces
# --------------------------------------------------------------------------

def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)).

    phi1 and phi2 of [NOTES] §2.1 are both SiLU. Written as z / (1 + e^{-z});
    for very negative z the denominator overflows to +inf and the value
    correctly tends to -0."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def time_bucket(dt, num_buckets: int = 32):
    """min(num_buckets - 1, floor(log2(|dt| + 1))) computed in integers.

    floor(log2(a)) for an integer a >= 1 is its bit length minus one, found
    here by repeated halving of the shift width (no floating point)."""
    a = np.abs(np.asarray(dt, dtype=np.int64)).astype(np.uint64) + np.uint64(1)
    r = np.zeros(a.shape, dtype=np.int64)
    for s in (32, 16, 8, 4, 2, 1):
        hi = (a >> np.uint64(s)) > 0
        a = np.where(hi, a >> np.uint64(s), a)
        r = r + np.where(hi, s, 0)
    return np.minimum(r, num_buckets - 1)


def genrank_bias(dp, dt, m_p: float, m_t: float, num_buckets: int = 32):
    """Parameter-free relative bias of [GENRANK] eq. 6.2.6:

        bias(i, j) = -m_p * (p_i - p_j) - m_t * bucket(t_i - t_j)

    with the slopes predefined (ALiBi-style, eq. 6.2.5, extended to time) and
    bucket() the same integer floor(log2(|dt| + 1)) bucketing as the table
    bias, so the two forms agree when the tables are filled linearly. m_p and
    m_t are scalars shared by all heads, as the equation prints them."""
    dp = np.asarray(dp, dtype=F64)
    return -m_p * dp - m_t * time_bucket(dt, num_buckets).astype(F64)


def stochastic_length(offsets, alpha: float, n_max: int, u, keys):
    """Stochastic Length ([GR-7.1] §7.1.5): a sequence of length n longer
    than N^(alpha/2) is, with probability p = 1 - N^alpha / n^2, replaced by
    a subsequence of k = floor(N^(alpha/2)) of its tokens; otherwise it is
    kept whole (N = n_max; alpha = 2 never truncates).

    The page prints N_{alpha/2} and N_alpha: read as powers. It says only
    that the subsequence is sampled; here the k tokens with the smallest
    keys are kept (ties to the earlier token), in their original order.
    Randomness comes in: u [B] uniform in [0, 1) decides truncation
    (truncate iff u_b < p_b); keys [T] rank the tokens. Everything is fp64.

    Returns (new offsets [B+1], source rows [T'] sequence-major)."""
    offsets = np.asarray(offsets, np.int64)
    u = np.asarray(u, np.float64)
    keys = np.asarray(keys, np.float64)
    N = float(n_max)
    k = int(np.floor(N ** (alpha / 2.0)))
    rows, lens = [], []
    for b in range(offsets.shape[0] - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        n = e - s
        keep = np.arange(s, e)
        if n > N ** (alpha / 2.0):
            p = 1.0 - N ** alpha / (float(n) * float(n))
            if u[b] < p:
                order = np.lexsort((np.arange(n), keys[s:e]))   # by key, then index
                keep = s + np.sort(order[:k])
        rows.append(keep)
        lens.append(keep.shape[0])
    new_off = np.zeros(len(lens) + 1, np.int64)
    np.cumsum(lens, out=new_off[1:])
    return new_off, (np.concatenate(rows) if rows else np.zeros(0, np.int64))


def layernorm(x, gamma, beta, eps: float):
    """LayerNorm over the d features of each token row, biased variance,
    affine gamma/beta (None: ones/zeros). Used for the optional input norm
    (Norm1) that the block diagram of [NOTES] §2.1 draws before f1."""
    x = np.asarray(x, F64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    n = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        n = n * np.asarray(gamma, F64)
    if beta is not None:
        n = n + np.asarray(beta, F64)
    return n


# --------------------------------------------------------------------------
# the three steps of the layer
# --------------------------------------------------------------------------

def proj(x, w1, b1, d: int):
    """Pointwise projection: U, V, Q, K = Split(SiLU(X W1^T + b1)).

    [NOTES] §2.1 first equation; [SA2HSTU] step 1. f1 is one linear layer
    (weight [4d, d] in out x in layout), phi1 = SiLU."""
    x = np.asarray(x, F64)
    z = x @ np.asarray(w1, F64).T
    if b1 is not None:
        z = z + np.asarray(b1, F64)
    h = silu(z)
    return h[:, 0:d], h[:, d:2 * d], h[:, 2 * d:3 * d], h[:, 3 * d:4 * d]


def _positions(L: int, m: int, n_cache: int) -> np.ndarray:
    """Positions of a sequence's own tokens: non-targets n_cache + j, all
    targets share n_cache + (L - m)."""
    p = n_cache + np.arange(L, dtype=np.int64)
    if m > 0:
        p[L - m:] = n_cache + (L - m)
    return p


def _visibility(L: int, m: int, n_cache: int, rows: np.ndarray, target_no_self: bool = False) -> np.ndarray:
    """Boolean [len(rows), n_cache + L] mask of visible keys for the given
    own-token query rows. target_no_self: a target (one of the last m
    tokens) does not see itself either, only the history and the
    non-targets (the literal reading of [GR-7.1] §7.1.5's M-FALCON: a
    candidate attends to the user history)."""
    j = np.arange(L)
    i = rows[:, None]
    self_ok = (j[None, :] == i) & ~(target_no_self & (i >= L - m))
    own = (j[None, :] <= i) & ((j[None, :] < L - m) | self_ok)
    cache = np.ones((rows.shape[0], n_cache), dtype=bool)
    return np.concatenate([cache, own], axis=1)


def attention(q, k, v, offsets, timestamps, pos_bias, time_bias, num_heads: int,
              n_max: int, alpha: float = 1.0, num_targets=None, cache=None,
              rows=None, row_chunk: int = 2048, linear_bias=None, num_time_buckets: int = 32,
              target_no_self: bool = False, token_types=None, num_token_types: int = 1):
    """Spatial aggregation, per head h of every sequence b:

        AV_h = (SiLU(alpha * Q_h K_h^T + rab_{p,t}) * Mask) V_h

    [NOTES] §2.1 second equation; [SA2HSTU] step 2; no softmax, no row
    normalisation ([GR-7.1] §7.1.4 innovation 1). rab and the mask as in the
    module docstring.

    q, k, v: [T, d] own tokens. offsets [B+1], timestamps [T].
    num_targets: None or int array [B] (last m_b tokens of b are targets).
    cache: None or dict(k=[Tc, d], v=[Tc, d], offsets=[B+1], timestamps=[Tc])
           holding keys/values visible to every query of the same sequence.
    rows: None (all tokens) or a sorted int array of global token rows; the
          result then has one row per requested token. Query rows are
          evaluated in chunks of ``row_chunk`` (each row's value is its own
          dense definition; chunking only bounds memory).
    linear_bias: None (rab from the tables), or (m_p, m_t): rab is then
          genrank_bias() of every pair, evaluated directly with
          ``num_time_buckets`` buckets; the tables are not used.
    target_no_self: targets do not see themselves (_visibility).
    token_types, num_token_types: the type-aware term of rab ([GR-7.1]
          §7.1.4, innovation 2: the bias is a function of the position
          difference, the time difference and the two tokens' types, so that
          different behaviours can decay at different rates). token_types
          [T] holds each own token's type in [0, nt); the cache dict then
          carries "types" [Tc]. time_bias is then nt * nt tables of nb
          buckets, flat: the pair (query type a, key type b) uses
          time_bias[(a * nt + b) * nb + bucket]; the position table stays
          shared. nt = 1 (or token_types None) is the untyped rab.
    Returns AV [T or len(rows), d] float64.
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    offsets = np.asarray(offsets, np.int64)
    timestamps = np.asarray(timestamps, np.int64)
    if linear_bias is None:
        pos_bias = np.asarray(pos_bias, F64)
        time_bias = np.asarray(time_bias, F64)
    T, d = q.shape
    dh = d // num_heads
    B = offsets.shape[0] - 1
    want = np.arange(T) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((want.shape[0], d), dtype=F64)
    nt = int(num_token_types) if token_types is not None else 1
    if nt < 1:
        raise ValueError("num_token_types must be >= 1")
    if linear_bias is not None:
        nb = num_time_buckets
    else:
        if time_bias.shape[0] % (nt * nt):
            raise ValueError("time_bias must hold num_token_types^2 tables")
        nb = time_bias.shape[0] // (nt * nt)
    types = None if token_types is None else np.asarray(token_types, np.int64)
    for b in range(B):
        s, e = int(offsets[b]), int(offsets[b + 1])
        L = e - s
        sel = np.nonzero((want >= s) & (want < e))[0]
        if L == 0 or sel.size == 0:
            continue
        m = 0 if num_targets is None else int(num_targets[b])
        if cache is not None:
            cs, ce = int(cache["offsets"][b]), int(cache["offsets"][b + 1])
            kc = np.asarray(cache["k"][cs:ce], F64)
            vc = np.asarray(cache["v"][cs:ce], F64)
            tc = np.asarray(cache["timestamps"][cs:ce], np.int64)
        else:
            cs = ce = 0
            kc = np.zeros((0, d))
            vc = np.zeros((0, d))
            tc = np.zeros(0, np.int64)
        nc = ce - cs
        if types is not None:
            ty_c = np.zeros(0, np.int64) if nc == 0 else np.asarray(cache["types"][cs:ce], np.int64)
            key_ty = np.concatenate([ty_c, types[s:e]])
        keys_k = np.concatenate([kc, k[s:e]], axis=0)
        keys_v = np.concatenate([vc, v[s:e]], axis=0)
        key_t = np.concatenate([tc, timestamps[s:e]])
        key_p = np.concatenate([np.arange(nc, dtype=np.int64), _positions(L, m, nc)])
        own_p = _positions(L, m, nc)
        for c0 in range(0, sel.size, row_chunk):
            csel = sel[c0:c0 + row_chunk]
            qrows = want[csel] - s                      # own-token indices
            dp = own_p[qrows][:, None] - key_p[None, :]
            dt = timestamps[s + qrows][:, None] - key_t[None, :]
            mask = _visibility(L, m, nc, qrows, target_no_self)
            if linear_bias is not None:
                rab = genrank_bias(dp, dt, linear_bias[0], linear_bias[1], nb)
            else:
                idx = dp + (n_max - 1)
                if np.any(mask & ((idx < 0) | (idx >= pos_bias.shape[0]))):
                    raise ValueError("position difference outside the position table")
                idx = np.clip(idx, 0, pos_bias.shape[0] - 1)
                tbi = time_bucket(dt, nb)
                if types is not None:
                    if np.any((types[s + qrows] < 0) | (types[s + qrows] >= nt)) or \
                            np.any((key_ty < 0) | (key_ty >= nt)):
                        raise ValueError("token type outside [0, num_token_types)")
                    tbi = (types[s + qrows][:, None] * nt + key_ty[None, :]) * nb + tbi
                rab = pos_bias[idx] + time_bias[tbi]
            for h in range(num_heads):
                cols = slice(h * dh, (h + 1) * dh)
                scores = alpha * (q[s + qrows, cols] @ keys_k[:, cols].T) + rab
                a = np.where(mask, silu(scores), 0.0)
                out[csel, cols] = a @ keys_v[:, cols]
    return out


def norm_gate(av, u, gamma, beta, eps: float):
    """G = (LayerNorm(AV) * gamma + beta) (.) U.

    [NOTES] §2.1 third equation and block diagram (LayerNorm, then the
    product with U); [SA2HSTU] step 3. LayerNorm over all d features of the
    token with the biased variance."""
    av = np.asarray(av, F64)
    mu = av.mean(axis=1, keepdims=True)
    var = ((av - mu) ** 2).mean(axis=1, keepdims=True)
    n = (av - mu) / np.sqrt(var + eps)
    if gamma is not None:
        n = n * np.asarray(gamma, F64)
    if beta is not None:
        n = n + np.asarray(beta, F64)
    return n * np.asarray(u, F64)


def output(x, g, w2, b2):
    """Y = X + G W2^T + b2: f2 is one linear layer ([NOTES] §2.1 third
    equation) and the residual from the input is the block diagram's skip
    connection."""
    y = np.asarray(x, F64) + np.asarray(g, F64) @ np.asarray(w2, F64).T
    if b2 is not None:
        y = y + np.asarray(b2, F64)
    return y


def _needed_prefix_rows(offsets, rows):
    """Global rows whose projections the requested query rows depend on: for
    each sequence, its prefix up to the last requested row."""
    offsets = np.asarray(offsets, np.int64)
    need = []
    for b in range(offsets.shape[0] - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        r = rows[(rows >= s) & (rows < e)]
        if r.size:
            need.append(np.arange(s, int(r.max()) + 1))
    return np.concatenate(need) if need else np.zeros(0, np.int64)


def layer(x, p, offsets, timestamps, num_heads: int, n_max: int, alpha: float = 1.0,
          eps: float = 1e-5, num_targets=None, cache=None, rows=None, token_types=None,
          num_token_types: int = 1) -> Dict[str, np.ndarray]:
    """One HSTU layer: projection, spatial aggregation, pointwise
    transformation ([NOTES] §2.1, all three equations, plus the residual).

    ``p`` has attributes w1, b1, w2, b2, gamma, beta, pos_bias, time_bias.
    Optional attributes: ``ln1_gamma``/``ln1_beta`` with ``input_norm`` true
    apply the input LayerNorm (Norm1 of the block diagram) to X before f1,
    while the residual keeps the raw X (the skip connection leaves from the
    input, ahead of Norm1); ``linear_bias`` = (m_p, m_t) replaces the table
    rab by genrank_bias().
    With ``rows`` given, only those token rows are produced (their causal
    prefixes are projected as needed). Returns a dict with u, v, q, k (for
    the projected rows ``proj_rows``), av, g and y (for the output rows)."""
    x = np.asarray(x, F64)
    offsets = np.asarray(offsets, np.int64)
    T, d = x.shape
    if rows is None:
        prow = np.arange(T)
        orow = np.arange(T)
    else:
        orow = np.asarray(rows, np.int64)
        prow = _needed_prefix_rows(offsets, orow)
    u = np.zeros((T, d)); vv = np.zeros((T, d)); qq = np.zeros((T, d)); kk = np.zeros((T, d))
    xin = x[prow]
    if getattr(p, "input_norm", False):
        xin = layernorm(xin, getattr(p, "ln1_gamma", None), getattr(p, "ln1_beta", None), eps)
    pu, pv, pq, pk = proj(xin, p.w1, p.b1, d)
    u[prow], vv[prow], qq[prow], kk[prow] = pu, pv, pq, pk
    lin = getattr(p, "linear_bias", None)
    nt = int(num_token_types) if token_types is not None else 1
    av = attention(qq, kk, vv, offsets, timestamps, p.pos_bias, p.time_bias, num_heads,
                   n_max, alpha, num_targets=num_targets, cache=cache,
                   rows=None if rows is None else orow, linear_bias=lin,
                   num_time_buckets=len(p.time_bias) // (nt * nt) if p.time_bias is not None else 32,
                   token_types=token_types, num_token_types=nt)
    g = norm_gate(av, u[orow], p.gamma, p.beta, eps)
    y = output(x[orow], g, p.w2, p.b2)
    return dict(u=u, v=vv, q=qq, k=kk, av=av, g=g, y=y, proj_rows=prow, rows=orow)


def silu_grad(z):
    """d SiLU / dz = s (1 + z (1 - s)), s = sigmoid(z)."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def silu_grad2(z):
    """d^2 SiLU / dz^2 = s (1 - s) (2 + z (1 - 2 s)), s = sigmoid(z)."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


def layer_backward(x, p, offsets, timestamps, dy, num_heads: int, n_max: int,
                   alpha: float = 1.0, eps: float = 1e-5,
                   magnitudes: bool = False) -> Dict[str, np.ndarray]:
    """Gradients of <Y, dY> for one layer with plain causal attention (no
    targets, no cache), the generative-training setting of [GR-7.1] §7.1.5:
    dX, dW1, db1, dW2, db2, dgamma, dbeta and the gradients of the position
    and time tables (the shared rab: every pair adds its score gradient,
    summed over heads, to the entry it read); with ``p.input_norm`` also
    dln1_gamma and dln1_beta of the input LayerNorm. The chain rule applied to the
    forward of layer() step by step, in float64.

    With ``magnitudes``, the result also holds ``mag``: for each vector
    gradient, the sum of the absolute values of the terms it adds up (the
    scale of the rounding error of a sum whose terms are computed in lower
    precision). The terms are the rows summed over tokens for db1, db2,
    dgamma, dbeta, dln1_gamma and dln1_beta. For the two tables a pair's
    term is its score gradient dS = SiLU'(S) dP with dP = dAV_i . V_j and
    S = alpha Q_i . K_j + rab, two dot products over the head's dh features;
    its magnitude is the first-order change of dS when every product in
    those dot products moves by its own size:
    |SiLU'(S)| (|dAV_i| . |V_j|) + |SiLU''(S)| |dP| |alpha| (|Q_i| . |K_j|).
    Test scaffolding: not a gradient."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    offsets = np.asarray(offsets, np.int64)
    timestamps = np.asarray(timestamps, np.int64)
    T, d = x.shape
    dh = d // num_heads
    w1, w2 = np.asarray(p.w1, F64), np.asarray(p.w2, F64)
    gamma = np.ones(d) if p.gamma is None else np.asarray(p.gamma, F64)
    beta = np.zeros(d) if p.beta is None else np.asarray(p.beta, F64)
    pb, tb = np.asarray(p.pos_bias, F64), np.asarray(p.time_bias, F64)
    nb = tb.shape[0]
    # forward, keeping what the backward needs
    norm1 = bool(getattr(p, "input_norm", False))
    xin = x
    if norm1:
        # the input LayerNorm (Norm1 of [NOTES] §2.1's block diagram) before f1
        g1 = getattr(p, "ln1_gamma", None)
        g1 = np.ones(d) if g1 is None else np.asarray(g1, F64)
        mu1 = x.mean(axis=1, keepdims=True)
        rstd1 = 1.0 / np.sqrt(((x - mu1) ** 2).mean(axis=1, keepdims=True) + eps)
        xhat1 = (x - mu1) * rstd1
        xin = layernorm(x, getattr(p, "ln1_gamma", None), getattr(p, "ln1_beta", None), eps)
    z = xin @ w1.T + (0.0 if p.b1 is None else np.asarray(p.b1, F64))
    h = silu(z)
    u, v, q, k = h[:, :d], h[:, d:2 * d], h[:, 2 * d:3 * d], h[:, 3 * d:]
    av = np.zeros((T, d))
    dq, dk, dv = np.zeros((T, d)), np.zeros((T, d)), np.zeros((T, d))
    dpos, dtime = np.zeros_like(pb), np.zeros_like(tb)
    mpos, mtime = np.zeros_like(pb), np.zeros_like(tb)
    seqs = []
    for b in range(offsets.shape[0] - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        if e == s:
            continue
        L = e - s
        i = np.arange(L)
        dp = i[:, None] - i[None, :]
        dt = timestamps[s:e][:, None] - timestamps[s:e][None, :]
        idx = np.clip(dp + (n_max - 1), 0, pb.shape[0] - 1)
        bkt = time_bucket(dt, nb)
        rab = pb[idx] + tb[bkt]
        mask = dp >= 0
        seqs.append((s, e, idx, bkt, rab, mask))
        for hh in range(num_heads):
            c = slice(hh * dh, (hh + 1) * dh)
            sc = alpha * (q[s:e, c] @ k[s:e, c].T) + rab
            av[s:e, c] = np.where(mask, silu(sc), 0.0) @ v[s:e, c]
    mu = av.mean(axis=1, keepdims=True)
    var = ((av - mu) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    nhat = (av - mu) * rstd
    nrm = nhat * gamma + beta
    g = nrm * u
    # Y = X + G W2^T + b2
    dg = dy @ w2
    dw2 = dy.T @ g
    db2 = dy.sum(axis=0)
    # G = (nhat gamma + beta) * U
    du = dg * nrm
    dnrm = dg * u
    dgamma = (dnrm * nhat).sum(axis=0)
    dbeta = dnrm.sum(axis=0)
    dnh = dnrm * gamma
    dav = rstd * (dnh - dnh.mean(axis=1, keepdims=True)
                  - nhat * (dnh * nhat).mean(axis=1, keepdims=True))
    # AV_h = (SiLU(S_h) * Mask) V_h, S_h = alpha Q_h K_h^T + rab
    for (s, e, idx, bkt, rab, mask) in seqs:
        for hh in range(num_heads):
            c = slice(hh * dh, (hh + 1) * dh)
            sc = alpha * (q[s:e, c] @ k[s:e, c].T) + rab
            pm = np.where(mask, silu(sc), 0.0)
            dv[s:e, c] += pm.T @ dav[s:e, c]
            dpm = dav[s:e, c] @ v[s:e, c].T
            ds = np.where(mask, dpm * silu_grad(sc), 0.0)
            dq[s:e, c] += alpha * (ds @ k[s:e, c])
            dk[s:e, c] += alpha * (ds.T @ q[s:e, c])
            np.add.at(dpos, idx[mask], ds[mask])
            np.add.at(dtime, bkt[mask], ds[mask])
            if magnitudes:
                mds = (np.abs(silu_grad(sc)) * (np.abs(dav[s:e, c]) @ np.abs(v[s:e, c]).T)
                       + np.abs(silu_grad2(sc)) * np.abs(dpm) * abs(alpha)
                       * (np.abs(q[s:e, c]) @ np.abs(k[s:e, c]).T))
                np.add.at(mpos, idx[mask], mds[mask])
                np.add.at(mtime, bkt[mask], mds[mask])
    # U, V, Q, K = Split(SiLU(Z)), Z = X W1^T + b1
    dz = np.concatenate([du, dv, dq, dk], axis=1) * silu_grad(z)
    dw1 = dz.T @ xin
    db1 = dz.sum(axis=0)
    dxin = dz @ w1
    extra = {}
    mag = dict(db1=np.abs(dz).sum(axis=0), db2=np.abs(dy).sum(axis=0),
               dgamma=np.abs(dnrm * nhat).sum(axis=0), dbeta=np.abs(dnrm).sum(axis=0),
               dpos=mpos, dtime=mtime)
    if norm1:
        # xin = xhat1 gamma1 + beta1, xhat1 = (x - mean) / sigma over the d features
        extra["dln1_gamma"] = (dxin * xhat1).sum(axis=0)
        extra["dln1_beta"] = dxin.sum(axis=0)
        mag["dln1_gamma"] = np.abs(dxin * xhat1).sum(axis=0)
        mag["dln1_beta"] = np.abs(dxin).sum(axis=0)
        dxh = dxin * g1
        dxin = rstd1 * (dxh - dxh.mean(axis=1, keepdims=True)
                        - xhat1 * (dxh * xhat1).mean(axis=1, keepdims=True))
    dx = dy + dxin
    if magnitudes:
        extra["mag"] = mag
    return dict(**extra, dx=dx, dw1=dw1, db1=db1, dw2=dw2, db2=db2, dgamma=dgamma, dbeta=dbeta,
                dpos=dpos, dtime=dtime)


def stack(x, layers: Sequence, offsets, timestamps, num_heads: int, n_max: int,
          alpha: float = 1.0, eps: float = 1e-5, return_all: bool = False):
    """L stacked layers: layer l's output is layer l+1's input ([GR-7.1]
    §7.1.6 scales depth; [NOTES] §2.1 defines one layer)."""
    h = np.asarray(x, F64)
    outs = [h]
    for p in layers:
        h = layer(h, p, offsets, timestamps, num_heads, n_max, alpha, eps)["y"]
        outs.append(h)
    return outs if return_all else h


def embed(item_emb, action_emb, item_ids, actions):
    """Action-oriented token: e_i = phi(x_i) + varphi(a_i), item embedding
    plus action embedding ([GENRANK] §6.2.2, eq. 6.2.2)."""
    return (np.asarray(item_emb, F64)[np.asarray(item_ids)] +
            np.asarray(action_emb, F64)[np.asarray(actions)])


# --------------------------------------------------------------------------
# ranking inference over a cached history (M-FALCON)
# --------------------------------------------------------------------------

def ranking(w, b_m: Optional[int] = None, eps: Optional[float] = None) -> Dict[str, List]:
    """Candidate scoring with micro-batches over a cached history, following
    [GR-7.1] §7.1.5 (M-FALCON: batched candidates with a mask, micro-batches,
    history K/V computed once and reused by every micro-batch).

    1. The history runs causally through every layer; layer l keeps K_l, V_l.
    2. Candidates are cut per user into micro-batches of b_m. Each
       micro-batch runs through the layers; at layer l its own tokens are all
       targets and the cache is (K_l, V_l) of the history.

    ``w`` is a ranking workload (``hstu_inputs.gen.make_ranking``). Returns
    dict(hist_y=[per layer outputs], cand_y=[T_cand, d] final candidate
    outputs in cand_x row order)."""
    from hstu_inputs.gen import micro_batches  # input layout only
    eps = w.ln_eps if eps is None else eps
    x = np.asarray(w.x, F64)
    caches = []
    hist_out = [x]
    for p in w.layers:
        r = layer(x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, eps)
        caches.append(dict(k=r["k"], v=r["v"], offsets=w.offsets, timestamps=w.timestamps))
        x = r["y"]
        hist_out.append(x)
    cand_y = np.zeros((int(w.cand_offsets[-1]), w.d_model))
    for offs, rws in micro_batches(w, b_m):
        xc = np.asarray(w.cand_x, F64)[rws]
        tc = np.asarray(w.cand_timestamps, np.int64)[rws]
        m = np.diff(offs)
        for l, p in enumerate(w.layers):
            xc = layer(xc, p, offs, tc, w.num_heads, w.n_max, w.alpha, eps,
                       num_targets=m, cache=caches[l])["y"]
        cand_y[rws] = xc
    return dict(hist_y=hist_out, cand_y=cand_y)


def ranking_independent(w, user: int, cand: int, eps: Optional[float] = None):
    """One candidate scored on its own: a plain causal forward over
    [history of ``user``, that one candidate] through every layer, no cache
    and no target mask. Returns the candidate's final output row. M-FALCON's
    batched, micro-batched and cached scoring must reproduce it ([GR-7.1]
    §7.1.5: batching changes the cost, not the per-candidate scores)."""
    eps = w.ln_eps if eps is None else eps
    s, e = int(w.offsets[user]), int(w.offsets[user + 1])
    c = int(w.cand_offsets[user]) + cand
    x = np.concatenate([np.asarray(w.x[s:e], F64), np.asarray(w.cand_x[c:c + 1], F64)])
    ts = np.concatenate([w.timestamps[s:e], w.cand_timestamps[c:c + 1]])
    offs = np.array([0, x.shape[0]], np.int64)
    for p in w.layers:
        x = layer(x, p, offs, ts, w.num_heads, w.n_max, w.alpha, eps)["y"]
    return x[-1]
