"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: brute force on tiny
inputs, independent library routines (scipy's expit, torch's layer_norm and
linear in float64), closed forms, invariants (causality, jagged-vs-padded,
head independence, linearity), the bucket definition in integers, and the
worked intensity example of the pointwise-aggregation section.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from hstu_inputs import gen

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _tiny(lengths, d=8, H=2, seed=0, affine="random", n_max=None, dtype="f32"):
    return gen.make_custom(lengths, d, H, dtype=dtype, seed=seed, affine=affine, n_max=n_max)


def _attn(w, q, k, v, p=None, **kw):
    p = p or w.layers[0]
    return oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias,
                            w.num_heads, w.n_max, w.alpha, **kw)


def _qkv(w, l=0):
    return oracle.proj(w.x, w.layers[l].w1, w.layers[l].b1, w.d_model)


def _brute_attention(q, k, v, offsets, ts, pb, tb, H, n_max, alpha, num_targets=None,
                     cache=None, types=None, nt=1):
    """Scalar triple loop straight from the definition (pure Python floats).
    With types: the time table is nt x nt tables of nb buckets (query type
    first)."""
    nb = len(tb) // (nt * nt)
    T, d = len(q), len(q[0])
    dh = d // H
    out = [[0.0] * d for _ in range(T)]
    for b in range(len(offsets) - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        L = e - s
        m = 0 if num_targets is None else int(num_targets[b])
        keys = []  # (k_row, v_row, position, timestamp, kind, own index)
        nc = 0
        if cache is not None:
            cs, ce = int(cache["offsets"][b]), int(cache["offsets"][b + 1])
            nc = ce - cs
            for c in range(nc):
                ty = int(cache["types"][cs + c]) if types is not None else 0
                keys.append((cache["k"][cs + c], cache["v"][cs + c], c,
                             int(cache["timestamps"][cs + c]), "cache", -1, ty))
        for j in range(L):
            pos = nc + (j if j < L - m else L - m)
            ty = int(types[s + j]) if types is not None else 0
            keys.append((k[s + j], v[s + j], pos, int(ts[s + j]), "own", j, ty))
        for i in range(L):
            p_i = nc + (i if i < L - m else L - m)
            t_i = int(ts[s + i])
            ty_i = int(types[s + i]) if types is not None else 0
            for (kr, vr, p_j, t_j, kind, j, ty_j) in keys:
                if kind == "own":
                    if j > i:
                        continue
                    if j >= L - m and j != i:
                        continue
                bucket = min(nb - 1, (abs(t_i - t_j) + 1).bit_length() - 1)
                rab = float(pb[p_i - p_j + n_max - 1]) + float(tb[(ty_i * nt + ty_j) * nb + bucket])
                for h in range(H):
                    dot = 0.0
                    for c in range(h * dh, (h + 1) * dh):
                        dot += float(q[s + i][c]) * float(kr[c])
                    sc = alpha * dot + rab
                    wgt = sc / (1.0 + math.exp(-sc)) if sc > -700 else 0.0
                    for c in range(h * dh, (h + 1) * dh):
                        out[s + i][c] += wgt * float(vr[c])
    return np.array(out)


# ---------------------------------------------------------------------------
# scalar pieces
# ---------------------------------------------------------------------------

def test_time_bucket_bruteforce_small():
    dt = np.arange(0, 1 << 20, dtype=np.int64)
    want = np.array([min(31, (int(a) + 1).bit_length() - 1) for a in dt[:5000]])
    assert np.array_equal(oracle.time_bucket(dt[:5000]), want)
    # full range against the integer definition via Python ints (vectorised
    # through a lookup of bit lengths per power-of-two band)
    got = oracle.time_bucket(dt)
    for kk in range(21):
        lo, hi = (1 << kk) - 1, (1 << (kk + 1)) - 1   # |dt|+1 in [2^k, 2^(k+1))
        band = got[lo:min(hi, dt.size)]
        assert np.all(band == min(kk, 31)), kk


def test_time_bucket_boundaries_and_clamp():
    for kk in range(1, 63):
        dt = (1 << kk) - 1  # |dt| + 1 == 2^k     -> bucket k
        assert oracle.time_bucket(np.array([dt]), 64)[0] == kk
        assert oracle.time_bucket(np.array([dt]))[0] == min(kk, 31)
        # |dt| + 1 == 2^k - 1 -> bucket k - 1;  |dt| + 1 == 2^k + 1 -> bucket k
        assert oracle.time_bucket(np.array([dt - 1]), 64)[0] == kk - 1
        assert oracle.time_bucket(np.array([dt + 1]), 64)[0] == kk
    assert oracle.time_bucket(np.array([0]))[0] == 0
    assert oracle.time_bucket(np.array([1]))[0] == 1
    assert oracle.time_bucket(np.array([2]))[0] == 1
    assert oracle.time_bucket(np.array([3]))[0] == 2
    # symmetric in the sign of dt, clamp at num_buckets-1
    x = np.array([-5, 5, -(1 << 40), (1 << 40)])
    assert list(oracle.time_bucket(x)) == [2, 2, 31, 31]
    assert list(oracle.time_bucket(x, num_buckets=8)) == [2, 2, 7, 7]


def test_silu_against_expit_and_identities():
    from scipy.special import expit
    z = np.linspace(-60, 60, 4001)
    np.testing.assert_allclose(oracle.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert oracle.silu(-1e4) == 0.0
    assert oracle.silu(1e4) == 1e4


# ---------------------------------------------------------------------------
# projection
# ---------------------------------------------------------------------------

def test_proj_against_torch_linear():
    import torch
    w = _tiny([5, 3], d=8, H=2, seed=3)
    p = w.layers[0]
    u, v, q, k = oracle.proj(w.x, p.w1, p.b1, 8)
    z = torch.nn.functional.linear(torch.tensor(w.x, dtype=torch.float64),
                                   torch.tensor(p.w1, dtype=torch.float64),
                                   torch.tensor(p.b1, dtype=torch.float64))
    h = torch.nn.functional.silu(z).numpy()
    np.testing.assert_allclose(np.concatenate([u, v, q, k], 1), h, rtol=1e-13, atol=1e-15)


def test_proj_bruteforce_and_split_order():
    w = _tiny([4], d=4, H=1, seed=4)
    p = w.layers[0]
    u, v, q, k = oracle.proj(w.x, p.w1, p.b1, 4)
    for t in range(4):
        for o in range(16):
            z = float(p.b1[o]) + sum(float(w.x[t][i]) * float(p.w1[o][i]) for i in range(4))
            want = z / (1 + math.exp(-z))
            got = [u, v, q, k][o // 4][t][o % 4]
            assert abs(got - want) < 1e-12
    # split order U, V, Q, K: W1 = 0 and chunk biases 1, 2, 3, 4
    b1 = np.repeat(np.arange(1.0, 5.0), 4)
    u, v, q, k = oracle.proj(w.x, np.zeros((16, 4)), b1, 4)
    for chunk, c in zip((u, v, q, k), (1.0, 2.0, 3.0, 4.0)):
        np.testing.assert_allclose(chunk, c / (1 + math.exp(-c)), rtol=1e-15)


def test_u_chunk_zero_gives_residual_plus_bias():
    w = _tiny([6, 4], d=8, H=2, seed=5)
    p = w.layers[0]
    p.w1[0:8] = 0.0
    p.b1[0:8] = 0.0
    r = oracle.layer(w.x, p, w.offsets, w.timestamps, 2, w.n_max)
    assert np.all(r["u"] == 0.0)
    np.testing.assert_allclose(r["y"], w.x.astype(np.float64) + p.b2.astype(np.float64), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,H,d", [([1], 1, 4), ([5, 1, 7], 2, 8), ([9, 16], 2, 4),
                                         ([0, 3, 0, 6], 2, 8)])
def test_attention_bruteforce(lengths, H, d):
    w = _tiny(lengths, d=d, H=H, seed=7, n_max=16)
    w.alpha = 0.7
    p = w.layers[0]
    # widen the time gaps so that many buckets are exercised
    w.timestamps = w.timestamps + np.arange(w.total_tokens) ** 3
    u, v, q, k = _qkv(w)
    got = _attn(w, q, k, v)
    want = _brute_attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias,
                            H, w.n_max, w.alpha)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_bruteforce_targets_and_cache():
    w = gen.make_ranking(seed=11, users=3, history=[4, 0, 6], candidates=[3, 2, 1],
                         micro_batch=2, d_model=8, num_heads=2, num_layers=1, affine="random",
                         dtype="f32")
    p = w.layers[0]
    rng = np.random.default_rng(0)
    hk = rng.standard_normal((w.total_tokens, 8))
    hv = rng.standard_normal((w.total_tokens, 8))
    cache = dict(k=hk, v=hv, offsets=w.offsets, timestamps=w.timestamps)
    cq = rng.standard_normal((int(w.cand_offsets[-1]), 8))
    ck = rng.standard_normal(cq.shape)
    cv = rng.standard_normal(cq.shape)
    # own tokens: 1 non-target followed by the rest as targets, per sequence
    m = np.maximum(np.diff(w.cand_offsets) - 1, 0)
    got = oracle.attention(cq, ck, cv, w.cand_offsets, w.cand_timestamps, p.pos_bias,
                           p.time_bias, 2, w.n_max, 1.0, num_targets=m, cache=cache)
    want = _brute_attention(cq, ck, cv, w.cand_offsets, w.cand_timestamps, p.pos_bias,
                            p.time_bias, 2, w.n_max, 1.0, num_targets=m, cache=cache)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_targets_without_self_closed_forms():
    """target_no_self: Q = K = 0 and rab == c. With no cache, a sequence of
    targets only sees nothing (AV = 0); with a cache, every target sees just
    the cache, AV = SiLU(c) * sum of the cache's V rows; non-targets keep
    their causal sums."""
    w = _tiny([5, 4], d=4, H=1, seed=3)
    p = w.layers[0]
    p.pos_bias[:] = 0.6
    p.time_bias[:] = 0.0
    c = float(p.pos_bias[0])      # the table's (float32) value
    z = np.zeros((w.total_tokens, 4))
    v = np.random.default_rng(4).standard_normal((w.total_tokens, 4))
    m = np.array([5, 2])          # sequence 0: all targets; sequence 1: 2 non-targets, 2 targets
    got = oracle.attention(z, z, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, 1, w.n_max,
                           num_targets=m, target_no_self=True)
    sc = c / (1 + math.exp(-c))
    assert np.all(got[0:5] == 0.0)
    np.testing.assert_allclose(got[5], sc * v[5], rtol=1e-14)
    np.testing.assert_allclose(got[6], sc * (v[5] + v[6]), rtol=1e-14)
    np.testing.assert_allclose(got[7], sc * (v[5] + v[6]), rtol=1e-14)   # targets: non-targets only
    np.testing.assert_allclose(got[8], sc * (v[5] + v[6]), rtol=1e-14)
    hv = np.random.default_rng(5).standard_normal((3, 4))
    cache = dict(k=np.zeros((3, 4)), v=hv, offsets=np.array([0, 3, 3]),
                 timestamps=np.array([1, 2, 3], np.int64))
    got = oracle.attention(z, z, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, 1, w.n_max,
                           num_targets=m, cache=cache, target_no_self=True)
    np.testing.assert_allclose(got[0:5], np.tile(sc * hv.sum(axis=0), (5, 1)), rtol=1e-14)


def test_attention_targets_without_self_drop_the_self_term():
    """A target's output without itself is its output with itself minus
    SiLU(S_ii) v_i, S_ii = alpha q_i.k_i + pos_bias[center] + time_bias[0]
    (targets share a position, and the time difference to itself is 0);
    other rows are unchanged."""
    w = _tiny([6, 7], d=8, H=2, seed=9, n_max=16)
    p = w.layers[0]
    u, v, q, k = _qkv(w)
    m = np.array([3, 7])
    a = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, 2, w.n_max,
                         alpha=0.8, num_targets=m)
    b = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, 2, w.n_max,
                         alpha=0.8, num_targets=m, target_no_self=True)
    targets = {3, 4, 5} | set(range(6, 13))
    for i in range(w.total_tokens):
        if i not in targets:
            np.testing.assert_array_equal(a[i], b[i])
            continue
        for h in range(2):
            cols = slice(4 * h, 4 * h + 4)
            s_ii = 0.8 * float(np.dot(q[i, cols], k[i, cols])) + float(p.pos_bias[w.n_max - 1]) + float(p.time_bias[0])
            self_term = s_ii / (1 + math.exp(-s_ii)) * v[i, cols]
            np.testing.assert_allclose(b[i, cols], a[i, cols] - self_term, rtol=1e-12, atol=1e-12)


def test_attention_closed_form_zero():
    w = _tiny([7, 3], d=8, H=2)
    p = w.layers[0]
    p.pos_bias[:] = 0.0
    p.time_bias[:] = 0.0
    z = np.zeros((w.total_tokens, 8))
    v = np.random.default_rng(1).standard_normal((w.total_tokens, 8))
    assert np.all(_attn(w, z, z, v) == 0.0)


def test_attention_closed_form_cumsum():
    """Q = K = 0 and rab == c: AV_i = SiLU(c) * sum_{j<=i} v_j (weights sum
    to (i+1) SiLU(c), more than 1: no normalisation)."""
    w = _tiny([9, 4], d=8, H=2)
    p = w.layers[0]
    c = 0.375
    p.pos_bias[:] = c
    p.time_bias[:] = 0.0
    z = np.zeros((w.total_tokens, 8))
    v = np.random.default_rng(2).standard_normal((w.total_tokens, 8))
    got = _attn(w, z, z, v)
    sc = c / (1 + math.exp(-c))
    for b in range(2):
        s, e = w.offsets[b], w.offsets[b + 1]
        np.testing.assert_allclose(got[s:e], sc * np.cumsum(v[s:e], axis=0), rtol=1e-13)


def test_attention_closed_form_position_convolution():
    """Q = K = 0, time table 0: AV = causal convolution of V with the kernel
    SiLU(pos_bias[n_max - 1 + lag])."""
    L = 12
    w = _tiny([L], d=4, H=1, n_max=L)
    p = w.layers[0]
    p.time_bias[:] = 0.0
    z = np.zeros((L, 4))
    v = np.random.default_rng(3).standard_normal((L, 4))
    got = _attn(w, z, z, v)
    kern = oracle.silu(p.pos_bias.astype(np.float64)[L - 1:2 * L - 1])
    for f in range(4):
        np.testing.assert_allclose(got[:, f], np.convolve(v[:, f], kern)[:L], rtol=1e-12,
                                   atol=1e-14)


def test_attention_closed_form_time_convolution():
    """Q = K = 0, pos table 0, timestamps t_j = t0 + j: the weight of lag k
    is SiLU(time_bias[bit_length(k + 1) - 1])."""
    L = 40
    w = _tiny([L], d=4, H=1, n_max=L)
    p = w.layers[0]
    p.pos_bias[:] = 0.0
    w.timestamps = 1_600_000_000 + np.arange(L, dtype=np.int64)
    z = np.zeros((L, 4))
    v = np.random.default_rng(4).standard_normal((L, 4))
    got = _attn(w, z, z, v)
    kern = np.array([p.time_bias[(lag + 1).bit_length() - 1] for lag in range(L)], np.float64)
    kern = oracle.silu(kern)
    for f in range(4):
        np.testing.assert_allclose(got[:, f], np.convolve(v[:, f], kern)[:L], rtol=1e-12,
                                   atol=1e-14)


def test_attention_genrank_linear_tables():
    """Tables filled linearly reproduce the parameter-free position/time bias
    -m_p (p_i - p_j) - m_t bucket(t_i - t_j) (GenRank eq. 6.2.6)."""
    L, mp, mt = 10, 0.0625, 0.25
    w = _tiny([L], d=4, H=1, n_max=L)
    p = w.layers[0]
    p.pos_bias[:] = -mp * (np.arange(2 * L - 1) - (L - 1))
    p.time_bias[:] = -mt * np.arange(32)
    w.timestamps = 1_600_000_000 + np.array([0, 1, 3, 7, 100, 101, 5000, 5001, 90000, 90003])
    z = np.zeros((L, 4))
    v = np.random.default_rng(5).standard_normal((L, 4))
    got = _attn(w, z, z, v)
    want = np.zeros((L, 4))
    for i in range(L):
        for j in range(i + 1):
            dt = int(w.timestamps[i] - w.timestamps[j])
            bias = -mp * (i - j) - mt * ((dt + 1).bit_length() - 1)
            want[i] += bias / (1 + math.exp(-bias)) * v[j]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_attention_single_token():
    w = _tiny([1], d=8, H=2, n_max=4)
    p = w.layers[0]
    u, v, q, k = _qkv(w)
    got = _attn(w, q, k, v)
    for h in range(2):
        c = slice(4 * h, 4 * h + 4)
        s = float(q[0, c] @ k[0, c]) + float(p.pos_bias[3]) + float(p.time_bias[0])
        np.testing.assert_allclose(got[0, c], s / (1 + math.exp(-s)) * v[0, c], rtol=1e-13)


def test_attention_causality():
    w = _tiny([14, 9], d=8, H=2)
    u, v, q, k = _qkv(w)
    base = _attn(w, q, k, v)
    rng = np.random.default_rng(6)
    for kk in (0, 5, 13):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for a in (q2, k2, v2):
            a[kk] += rng.standard_normal(8)
        out = _attn(w, q2, k2, v2)
        np.testing.assert_array_equal(out[:kk], base[:kk])
        np.testing.assert_array_equal(out[14:], base[14:])  # other sequence untouched
        assert not np.allclose(out[kk], base[kk])


def test_layer_causality():
    w = _tiny([12, 6], d=8, H=2)
    p = w.layers[0]
    base = oracle.layer(w.x, p, w.offsets, w.timestamps, 2, w.n_max)["y"]
    x2 = w.x.copy()
    x2[7] += 1.0
    ts2 = w.timestamps.copy()
    ts2[9] += 1234  # later timestamp only affects rows >= 9
    out = oracle.layer(x2, p, w.offsets, ts2, 2, w.n_max)["y"]
    np.testing.assert_array_equal(out[:7], base[:7])
    np.testing.assert_array_equal(out[12:], base[12:])


def test_jagged_equals_per_sequence_and_padded():
    lengths = [5, 1, 8, 3]
    w = _tiny(lengths, d=8, H=2, n_max=12)
    p = w.layers[0]
    full = oracle.layer(w.x, p, w.offsets, w.timestamps, 2, w.n_max)["y"]
    rng = np.random.default_rng(7)
    for b, L in enumerate(lengths):
        s, e = w.offsets[b], w.offsets[b + 1]
        one = oracle.layer(w.x[s:e], p, np.array([0, L]), w.timestamps[s:e], 2, w.n_max)["y"]
        np.testing.assert_allclose(one, full[s:e], rtol=1e-13, atol=1e-14)
        # padded to 12 with garbage tokens at the end: the first L rows stay
        pad = 12 - L
        xp = np.concatenate([w.x[s:e], rng.standard_normal((pad, 8))])
        tp = np.concatenate([w.timestamps[s:e],
                             w.timestamps[e - 1] + 1 + np.arange(pad, dtype=np.int64)])
        padded = oracle.layer(xp, p, np.array([0, 12]), tp, 2, w.n_max)["y"]
        np.testing.assert_allclose(padded[:L], full[s:e], rtol=1e-13, atol=1e-14)


def test_attention_structure_linearity_heads_permutation():
    w = _tiny([6, 4, 5], d=8, H=2)
    u, v, q, k = _qkv(w)
    base = _attn(w, q, k, v)
    rng = np.random.default_rng(8)
    v2 = rng.standard_normal(v.shape)
    np.testing.assert_allclose(_attn(w, q, k, 2.0 * v - 3.0 * v2),
                               2.0 * base - 3.0 * _attn(w, q, k, v2), rtol=1e-11, atol=1e-12)
    # head independence: change head 1's inputs, head 0 is untouched
    q3, k3 = q.copy(), k.copy()
    q3[:, 4:] += 1.0
    k3[:, 4:] -= 0.5
    out = _attn(w, q3, k3, v)
    np.testing.assert_array_equal(out[:, :4], base[:, :4])
    assert not np.allclose(out[:, 4:], base[:, 4:])
    # permuting sequences permutes outputs
    order = [2, 0, 1]
    segs = [np.arange(w.offsets[b], w.offsets[b + 1]) for b in order]
    perm = np.concatenate(segs)
    offs = gen.make_jagged([len(s) for s in segs])
    p = w.layers[0]
    out = oracle.attention(q[perm], k[perm], v[perm], offs, w.timestamps[perm], p.pos_bias,
                           p.time_bias, 2, w.n_max)
    np.testing.assert_allclose(out, base[perm], rtol=1e-14, atol=1e-15)


def test_attention_rows_subset_matches_full():
    w = _tiny([7, 11, 2], d=8, H=2)
    u, v, q, k = _qkv(w)
    base = _attn(w, q, k, v)
    rows = np.array([0, 3, 8, 17, 19])
    np.testing.assert_allclose(_attn(w, q, k, v, rows=rows), base[rows], rtol=1e-14)
    full = oracle.layer(w.x, w.layers[0], w.offsets, w.timestamps, 2, w.n_max)
    part = oracle.layer(w.x, w.layers[0], w.offsets, w.timestamps, 2, w.n_max, rows=rows)
    np.testing.assert_allclose(part["y"], full["y"][rows], rtol=1e-13, atol=1e-14)


def test_pos_table_range_error():
    w = _tiny([6], d=4, H=1, n_max=3)
    u, v, q, k = _qkv(w)
    with pytest.raises(ValueError):
        _attn(w, q, k, v)


def test_golden_intensity_example():
    """Worked example of the pointwise-aggregation section: softmax gives
    users A and B the same split; SiLU aggregation keeps B's 10x
    intensity."""
    g = json.load(open(os.path.join(HERE, "golden", "intensity_example.json")))
    c = 0.75
    outs = {}
    for name, cnt in g["users"].items():
        L = cnt["tech"] + cnt["ent"] + 1
        w = _tiny([L], d=2, H=1, n_max=L)
        p = w.layers[0]
        p.pos_bias[:] = c
        p.time_bias[:] = 0.0
        v = np.zeros((L, 2))
        v[:cnt["tech"], 0] = 1.0
        v[cnt["tech"]:L - 1, 1] = 1.0
        z = np.zeros((L, 2))
        outs[name] = _attn(w, z, z, v)[L - 1]
        sc = c / (1 + math.exp(-c))
        np.testing.assert_allclose(outs[name] / sc, g["pointwise_counts_over_silu_c"][name],
                                   rtol=1e-13)
        split = outs[name] / outs[name].sum()
        np.testing.assert_allclose(split, g["softmax_split"], rtol=1e-12)
    np.testing.assert_allclose(outs["B"], 10.0 * outs["A"], rtol=1e-13)


# ---------------------------------------------------------------------------
# pointwise transformation
# ---------------------------------------------------------------------------

def test_norm_gate_against_torch_layer_norm():
    import torch
    rng = np.random.default_rng(9)
    av = rng.standard_normal((7, 16)) * 3 + 5
    u = rng.standard_normal((7, 16))
    gm = 1 + 0.1 * rng.standard_normal(16)
    bt = 0.1 * rng.standard_normal(16)
    ln = torch.nn.functional.layer_norm(torch.tensor(av), (16,), torch.tensor(gm),
                                        torch.tensor(bt), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.norm_gate(av, u, gm, bt, 1e-5), ln * u, rtol=1e-12,
                               atol=1e-13)


def test_norm_gate_moments_and_scale_invariance():
    rng = np.random.default_rng(10)
    av = rng.standard_normal((5, 32)) + 4
    ones = np.ones((5, 32))
    g = oracle.norm_gate(av, ones, np.full(32, 2.0), np.full(32, 0.5), 0.0)
    np.testing.assert_allclose(g.mean(axis=1), 0.5, rtol=1e-12)
    np.testing.assert_allclose(g.var(axis=1), 4.0, rtol=1e-12)
    np.testing.assert_allclose(oracle.norm_gate(7.5 * av, ones, None, None, 0.0),
                               oracle.norm_gate(av, ones, None, None, 0.0), rtol=1e-12)


def test_output_closed_forms():
    w = _tiny([5], d=8, H=2, seed=12)
    p = w.layers[0]
    p.w2[:] = 0.0
    r = oracle.layer(w.x, p, w.offsets, w.timestamps, 2, w.n_max)
    np.testing.assert_allclose(r["y"], w.x.astype(np.float64) + p.b2.astype(np.float64), rtol=0, atol=1e-15)
    # V scaled by c leaves Y unchanged when eps = 0 (LayerNorm scale invariance)
    w = _tiny([6], d=8, H=2, seed=13)
    p = w.layers[0]
    y0 = oracle.layer(w.x, p, w.offsets, w.timestamps, 2, w.n_max, eps=0.0)["y"]
    u, v, q, k = _qkv(w)
    av = _attn(w, q, k, 3.0 * v)
    y1 = oracle.output(w.x, oracle.norm_gate(av, u, p.gamma, p.beta, 0.0), p.w2, p.b2)
    np.testing.assert_allclose(y1, y0, rtol=1e-11, atol=1e-12)


def test_output_bruteforce():
    rng = np.random.default_rng(14)
    x, g = rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    w2, b2 = rng.standard_normal((4, 4)), rng.standard_normal(4)
    y = oracle.output(x, g, w2, b2)
    for t in range(3):
        for o in range(4):
            want = x[t][o] + b2[o] + sum(g[t][i] * w2[o][i] for i in range(4))
            assert abs(y[t][o] - want) < 1e-12


# ---------------------------------------------------------------------------
# stack, embedding, ranking
# ---------------------------------------------------------------------------

def test_stack_equals_chained_layers():
    w = gen.make_custom([5, 9], 8, 2, dtype="f32", seed=15, num_layers=3, affine="random")
    outs = oracle.stack(w.x, w.layers, w.offsets, w.timestamps, 2, w.n_max, return_all=True)
    h = w.x
    for l, p in enumerate(w.layers):
        h = oracle.layer(h, p, w.offsets, w.timestamps, 2, w.n_max)["y"]
        np.testing.assert_array_equal(outs[l + 1], h)


def test_embed_closed_form():
    item = np.arange(50, dtype=np.float64)[:, None] * np.ones((1, 4))
    act = 1000.0 * np.arange(16, dtype=np.float64)[:, None] * np.ones((1, 4))
    ids = np.array([3, 49, 0, 3])
    a = np.array([0, 15, 2, 7])
    x = oracle.embed(item, act, ids, a)
    np.testing.assert_array_equal(x[:, 0], ids + 1000.0 * a)
    np.testing.assert_array_equal(x[:, 3], ids + 1000.0 * a)


def _small_ranking(seed=21, history=(6, 3, 9), candidates=(5, 7, 2), layers=2):
    return gen.make_ranking(seed=seed, users=3, history=list(history),
                            candidates=list(candidates), micro_batch=2, d_model=8,
                            num_heads=2, num_layers=layers, affine="random", dtype="f32")


def test_ranking_equals_independent_forwards():
    w = _small_ranking()
    r = oracle.ranking(w)
    for u in range(3):
        for c in range(int(w.cand_offsets[u + 1] - w.cand_offsets[u])):
            want = oracle.ranking_independent(w, u, c)
            np.testing.assert_allclose(r["cand_y"][w.cand_offsets[u] + c], want, rtol=1e-11,
                                       atol=1e-12)


@pytest.mark.parametrize("b_m", [1, 3, 7, 512])
def test_ranking_microbatch_invariance(b_m):
    w = _small_ranking()
    full = oracle.ranking(w, b_m=512)["cand_y"]
    np.testing.assert_allclose(oracle.ranking(w, b_m=b_m)["cand_y"], full, rtol=1e-12,
                               atol=1e-13)


def test_history_pass_is_plain_stack():
    w = _small_ranking()
    r = oracle.ranking(w)
    outs = oracle.stack(w.x, w.layers, w.offsets, w.timestamps, w.num_heads, w.n_max,
                        return_all=True)
    for a, b in zip(r["hist_y"], outs):
        np.testing.assert_array_equal(a, b)


def test_generator_recipe():
    for k in (0, 1, 2):
        w = gen.make_config(k)
        L = w.lengths
        for b in range(w.num_seqs):
            t = w.timestamps[w.offsets[b]:w.offsets[b + 1]]
            assert t[0] == gen.T0_SECONDS and np.all(np.diff(t) >= 1)
        if k == 1:
            assert L.min() >= 16 and L.max() <= 512 and w.num_seqs == 64
        if k == 2:
            assert L[0] == 8192 and L.min() >= 2048 and w.num_seqs == 16
        assert w.layers[0].pos_bias.shape[0] == 2 * w.n_max - 1
        if w.dtype == "bf16":
            np.testing.assert_array_equal(gen.bf16_round(w.x), w.x)
            np.testing.assert_array_equal(gen.bf16_round(w.layers[0].w1), w.layers[0].w1)


# ---------------------------------------------------------------------------
# options: parameter-free bias (GenRank eq. 6.2.6) and the input LayerNorm
# ---------------------------------------------------------------------------

def test_genrank_bias_worked_example():
    """The worked example after GenRank eq. 6.2.6: the 7th, 5th and 1st of
    seven past interactions, seen from the 8th, carry a small, a medium and a
    large penalty. Any positive slopes must order them so; with m_t = 0 the
    bias is ALiBi's -m (i - j) (eq. 6.2.5)."""
    ex = json.load(open(os.path.join(HERE, "golden", "genrank_alibi_example.json")))
    items = ex["interactions"]
    assert [it["penalty"] for it in items] == ["small", "medium", "large"]
    dp = np.array([it["position_distance"] for it in items])
    dt = np.array([it["time_distance_s"] for it in items])
    # bucket = bit length of |dt| + 1, minus one: 301 -> 8, 3601 -> 11, 86401 -> 16
    assert list(oracle.time_bucket(dt)) == [8, 11, 16]
    for mp, mt in [(0.5, 0.25), (0.01, 1.0), (2.0, 0.0), (0.0, 0.1)]:
        b = oracle.genrank_bias(dp, dt, mp, mt)
        assert np.all(b <= 0)
        assert b[0] > b[1] > b[2]
        if mt == 0.0:
            np.testing.assert_array_equal(b, -mp * dp)


def _with_targets_and_cache(seed):
    w = _tiny([7, 1, 12, 5], d=8, H=2, seed=seed, n_max=24)
    rng = np.random.default_rng(seed + 100)
    q, k, v = (rng.standard_normal((int(w.offsets[-1]), 8)) for _ in range(3))
    nt = np.array([2, 0, 3, 5])
    coff = np.array([0, 3, 3, 9, 11])
    cache = dict(offsets=coff, k=rng.standard_normal((11, 8)), v=rng.standard_normal((11, 8)),
                 timestamps=1_500_000_000 + np.sort(rng.integers(0, 10**6, 11)))
    return w, q, k, v, nt, cache


def test_attention_linear_bias_matches_linear_tables():
    """The direct eq. 6.2.6 path equals the table path with tables filled
    linearly, with targets and a cache (two separate code paths)."""
    w, q, k, v, nt, cache = _with_targets_and_cache(3)
    mp, mt = 0.03125, 0.125
    p = w.layers[0]
    n = w.n_max
    pb = -mp * (np.arange(2 * n - 1) - (n - 1))
    tb = -mt * np.arange(32)
    a = oracle.attention(q, k, v, w.offsets, w.timestamps, pb, tb, 2, n, w.alpha,
                         num_targets=nt, cache=cache)
    b = oracle.attention(q, k, v, w.offsets, w.timestamps, None, None, 2, n, w.alpha,
                         num_targets=nt, cache=cache, linear_bias=(mp, mt))
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-13)
    c = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, 2, n,
                         w.alpha, num_targets=nt, cache=cache)
    assert not np.allclose(b, c)


def test_attention_linear_bias_shift_invariance():
    """Eq. 6.2.6 depends on differences only: shifting every timestamp (own
    and cached) by one constant leaves the output unchanged."""
    w, q, k, v, nt, cache = _with_targets_and_cache(4)
    kw = dict(num_targets=nt, linear_bias=(0.05, 0.2))
    a = oracle.attention(q, k, v, w.offsets, w.timestamps, None, None, 2, w.n_max, w.alpha,
                         cache=cache, **kw)
    c2 = dict(cache, timestamps=cache["timestamps"] + 86_400 * 365)
    b = oracle.attention(q, k, v, w.offsets, w.timestamps + 86_400 * 365, None, None, 2,
                         w.n_max, w.alpha, cache=c2, **kw)
    np.testing.assert_allclose(b, a, rtol=1e-14, atol=1e-14)


def test_layernorm_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((37, 24)) * 3 + 1.5
    g, b = rng.standard_normal(24), rng.standard_normal(24)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(g),
                                          torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layernorm(x, g, b, 1e-5), want, rtol=1e-12, atol=1e-12)


def _norm1_workload(seed, eps):
    w = _tiny([6, 9, 1], d=8, H=2, seed=seed, n_max=9)
    w.ln_eps = eps
    rng = np.random.default_rng(seed + 7)
    p = w.layers[0]
    p.input_norm = True
    p.ln1_gamma = 1.0 + 0.3 * rng.standard_normal(8)
    p.ln1_beta = 0.2 * rng.standard_normal(8)
    return w, p


def _layer_y(w, x, p):
    return oracle.layer(x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha,
                        w.ln_eps)["y"]


def test_layer_input_norm_residual_carries_raw_x():
    """With Norm1, f1 sees LN(X) but the skip connection carries X: the
    layer's update Y - X equals that of the plain layer run on LN(X)."""
    import copy
    w, p = _norm1_workload(5, 1e-5)
    x = np.asarray(w.x, np.float64) * 2.0 + 0.7
    y1 = _layer_y(w, x, p)
    plain = copy.copy(p)
    plain.input_norm = False
    xn = oracle.layernorm(x, p.ln1_gamma, p.ln1_beta, w.ln_eps)
    y0 = _layer_y(w, xn, plain)
    np.testing.assert_allclose(y1 - x, y0 - xn, rtol=1e-12, atol=1e-12)
    assert not np.allclose(y1, y0)


def test_layer_input_norm_scale_shift_invariance():
    """LayerNorm with eps = 0 ignores a positive scale and a shift of each
    row, so with Norm1 the layer's update Y - X does too."""
    w, p = _norm1_workload(6, 0.0)
    x = np.asarray(w.x, np.float64)
    base = _layer_y(w, x, p) - x
    x2 = 3.5 * x - 1.25
    np.testing.assert_allclose(_layer_y(w, x2, p) - x2, base, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------------------
# Stochastic Length ([GR-7.1] §7.1.5)
# ---------------------------------------------------------------------------

def test_stochastic_length_alpha_two_keeps_everything():
    """alpha = 2 degenerates to no truncation (stated on the page)."""
    rng = np.random.default_rng(1)
    off = gen.make_jagged([0, 1, 300, 4096, 8192])
    new_off, rows = oracle.stochastic_length(off, 2.0, 8192, rng.random(5), rng.random(int(off[-1])))
    np.testing.assert_array_equal(new_off, off)
    np.testing.assert_array_equal(rows, np.arange(int(off[-1])))


def test_stochastic_length_bruteforce_small():
    """Short sequences stay whole; a truncated one keeps exactly floor(N^(a/2))
    tokens, the ones with the smallest keys, in order (brute force over all
    subsets of a tiny sequence)."""
    import itertools
    N, alpha = 16, 1.5                       # N^(a/2) = 8, N^a = 64
    lens = [3, 8, 12]
    off = gen.make_jagged(lens)
    keys = np.array([0.5, 0.1, 0.9] + list(np.linspace(1, 0, 8)) +
                    [0.3, 0.8, 0.1, 0.7, 0.2, 0.95, 0.05, 0.6, 0.4, 0.85, 0.15, 0.5])
    u = np.array([0.0, 0.0, 0.0])           # truncate whenever allowed (p > 0)
    new_off, rows = oracle.stochastic_length(off, alpha, N, u, keys)
    assert list(np.diff(new_off)) == [3, 8, 8]   # 3, 8 <= 8 stay; 12 > 8, p = 1 - 64/144
    np.testing.assert_array_equal(rows[:11], np.arange(11))
    s = int(off[2])
    best = min(itertools.combinations(range(12), 8), key=lambda c: sum(keys[s + j] for j in c))
    np.testing.assert_array_equal(rows[11:], s + np.array(best))
    u_hi = np.array([0.0, 0.0, 1.0 - 64 / 144])   # u = p: not truncated (strict u < p)
    new_off, _ = oracle.stochastic_length(off, alpha, N, u_hi, keys)
    assert list(np.diff(new_off)) == [3, 8, 12]


def test_stochastic_length_frequency_matches_p():
    """Over many draws the truncation frequency of a length-n sequence is
    p = 1 - N^a / n^2 (binomial, 6 sigma)."""
    N, alpha, n, draws = 8192, 1.6, 4096, 20000
    off = gen.make_jagged([n] * draws)
    rng = np.random.default_rng(7)
    u = rng.random(draws)
    p = 1.0 - N ** alpha / n ** 2
    lens = []
    for b0 in range(0, draws, 2000):          # one call per block keeps keys small
        sub = gen.make_jagged([n] * 2000)
        new_off, _ = oracle.stochastic_length(sub, alpha, N, u[b0:b0 + 2000],
                                              np.zeros(int(sub[-1])))
        lens.extend(np.diff(new_off))
    frac = np.mean(np.asarray(lens) < n)
    assert abs(frac - p) < 6 * math.sqrt(p * (1 - p) / draws), (frac, p)
    assert set(lens) <= {n, int(N ** (alpha / 2))}


# ---------------------------------------------------------------------------
# layer backward (generative training, plain causal attention)
# ---------------------------------------------------------------------------

def test_silu_grad_closed_form_and_difference():
    z = np.linspace(-30, 30, 241)
    h = 1e-6
    num = (oracle.silu(z + h) - oracle.silu(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.silu_grad(z), num, rtol=1e-6, atol=1e-9)
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5          # sigma(0) = 1/2
    np.testing.assert_allclose(oracle.silu_grad(np.array([60.0])), [1.0], atol=1e-20)


def _bwd_case(seed):
    w = _tiny([5, 1, 7, 0, 3], d=8, H=2, seed=seed, affine="random", n_max=7)
    w.alpha = 0.7
    rng = np.random.default_rng(seed + 1000)
    dy = rng.standard_normal((w.total_tokens, 8))
    return w, dy


def _f(w, x, p, dy):
    y = oracle.layer(x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, w.ln_eps)["y"]
    return float((y * dy).sum())


@pytest.mark.parametrize("name", ["x", "w1", "b1", "w2", "b2", "gamma", "beta", "pos_bias",
                                  "time_bias"])
def test_layer_backward_matches_central_differences(name):
    """<grad, v> equals the central difference of <Y, dY> along a random v,
    for every input and parameter: the forward oracle checks the backward."""
    import copy
    w, dy = _bwd_case(3)
    p = w.layers[0]
    x = np.asarray(w.x, np.float64)
    g = oracle.layer_backward(x, p, w.offsets, w.timestamps, dy, w.num_heads, w.n_max, w.alpha,
                              w.ln_eps)
    key = {"x": "dx", "w1": "dw1", "b1": "db1", "w2": "dw2", "b2": "db2", "gamma": "dgamma",
           "beta": "dbeta", "pos_bias": "dpos", "time_bias": "dtime"}[name]
    base = x if name == "x" else np.asarray(getattr(p, name), np.float64)
    v = np.random.default_rng(99).standard_normal(base.shape)
    eps = 1e-5

    def at(t):
        pp = copy.copy(p)
        xx = x
        if name == "x":
            xx = x + t * v
        else:
            setattr(pp, name, base + t * v)
        return _f(w, xx, pp, dy)

    num = (at(eps) - at(-eps)) / (2 * eps)
    ana = float((g[key] * v).sum())
    assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (name, num, ana)


@pytest.mark.parametrize("name", ["x", "w1", "ln1_gamma", "ln1_beta", "time_bias"])
def test_layer_backward_with_input_norm_matches_central_differences(name):
    """The same check with the input LayerNorm before f1 (its gamma and beta
    random): the gradient reaches X through the residual and through Norm1."""
    import copy
    w, dy = _bwd_case(5)
    p = copy.copy(w.layers[0])
    rng = np.random.default_rng(55)
    p.input_norm = True
    p.ln1_gamma = 1.0 + 0.3 * rng.standard_normal(8)
    p.ln1_beta = 0.2 * rng.standard_normal(8)
    x = np.asarray(w.x, np.float64)
    g = oracle.layer_backward(x, p, w.offsets, w.timestamps, dy, w.num_heads, w.n_max, w.alpha,
                              w.ln_eps)
    key = {"x": "dx", "w1": "dw1", "ln1_gamma": "dln1_gamma", "ln1_beta": "dln1_beta",
           "time_bias": "dtime"}[name]
    base = x if name == "x" else np.asarray(getattr(p, name), np.float64)
    v = np.random.default_rng(98).standard_normal(base.shape)
    eps = 1e-5

    def at(t):
        pp = copy.copy(p)
        xx = x
        if name == "x":
            xx = x + t * v
        else:
            setattr(pp, name, base + t * v)
        return _f(w, xx, pp, dy)

    num = (at(eps) - at(-eps)) / (2 * eps)
    ana = float((g[key] * v).sum())
    assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (name, num, ana)


def test_layer_backward_linear_in_dy_and_residual():
    """Gradients are linear in dY; with W2 = 0 the only path to X is the
    residual, so dX = dY and W1, b1, gamma, beta and the tables get nothing."""
    w, dy = _bwd_case(4)
    p = w.layers[0]
    x = np.asarray(w.x, np.float64)
    args = (w.offsets, w.timestamps)
    kw = dict(num_heads=w.num_heads, n_max=w.n_max, alpha=w.alpha, eps=w.ln_eps)
    g1 = oracle.layer_backward(x, p, *args, dy, **kw)
    g2 = oracle.layer_backward(x, p, *args, -2.5 * dy, **kw)
    for kk in g1:
        np.testing.assert_allclose(g2[kk], -2.5 * g1[kk], rtol=1e-12, atol=1e-12)
    import copy
    p0 = copy.copy(p)
    p0.w2 = np.zeros_like(p.w2)
    g0 = oracle.layer_backward(x, p0, *args, dy, **kw)
    np.testing.assert_array_equal(g0["dx"], dy)
    for kk in ("dw1", "db1", "dgamma", "dbeta", "dpos", "dtime"):
        assert np.all(g0[kk] == 0), kk


def test_silu_grad2_matches_central_differences():
    """SiLU'' against the central difference of SiLU', its value 1/2 at 0
    and its decay far from 0."""
    z = np.linspace(-12.0, 12.0, 97)
    h = 1e-5
    num = (oracle.silu_grad(z + h) - oracle.silu_grad(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.silu_grad2(z), num, rtol=1e-6, atol=1e-9)
    assert oracle.silu_grad2(np.array([0.0]))[0] == 0.5
    assert abs(oracle.silu_grad2(np.array([60.0]))[0]) < 1e-20


def _mag_case(seed, norm1):
    import copy
    w, dy = _bwd_case(seed)
    p = copy.copy(w.layers[0])
    if norm1:
        rng = np.random.default_rng(seed + 7)
        p.input_norm = True
        p.ln1_gamma = 1.0 + 0.3 * rng.standard_normal(8)
        p.ln1_beta = 0.2 * rng.standard_normal(8)
    return w, p, dy


@pytest.mark.parametrize("norm1", [False, True])
def test_backward_magnitudes_bound_and_balance(norm1):
    """The term magnitudes of the vector gradients: the gradients are the
    same with and without them; each entry is at most its magnitude
    (triangle inequality); every visible pair and head adds its magnitude to
    one entry of each table, so the two tables' magnitudes have equal sums;
    and they scale with |c| when dY is multiplied by c (every term is linear
    in dY)."""
    w, p, dy = _mag_case(11, norm1)
    x = np.asarray(w.x, np.float64)
    args = (x, p, w.offsets, w.timestamps)
    kw = dict(num_heads=w.num_heads, n_max=w.n_max, alpha=w.alpha, eps=w.ln_eps)
    g = oracle.layer_backward(*args, dy, **kw, magnitudes=True)
    plain = oracle.layer_backward(*args, dy, **kw)
    assert "mag" not in plain
    for k in plain:
        np.testing.assert_array_equal(g[k], plain[k])
    mag = g["mag"]
    names = ["db1", "db2", "dgamma", "dbeta", "dpos", "dtime"] + (["dln1_gamma", "dln1_beta"] if norm1 else [])
    assert sorted(mag) == sorted(names)
    for k in names:
        assert mag[k].shape == g[k].shape
        assert np.all(mag[k] >= np.abs(g[k]) * (1 - 1e-12)), k
    assert mag["dpos"].sum() > 0
    np.testing.assert_allclose(mag["dpos"].sum(), mag["dtime"].sum(), rtol=1e-12)
    g3 = oracle.layer_backward(*args, -3.0 * dy, **kw, magnitudes=True)
    for k in names:
        np.testing.assert_allclose(g3["mag"][k], 3.0 * mag[k], rtol=1e-12, atol=1e-300)


def test_backward_magnitudes_special_cases():
    """With dY >= 0 every term of db2 is non-negative, so its magnitude is
    db2 itself; with W2 = 0 no gradient reaches G's producers, and every
    magnitude but db2's is zero; with dY = 0 all are zero."""
    import copy
    w, p, dy = _mag_case(12, False)
    x = np.asarray(w.x, np.float64)
    kw = dict(num_heads=w.num_heads, n_max=w.n_max, alpha=w.alpha, eps=w.ln_eps, magnitudes=True)
    g = oracle.layer_backward(x, p, w.offsets, w.timestamps, np.abs(dy), **kw)
    np.testing.assert_allclose(g["mag"]["db2"], g["db2"], rtol=1e-12)
    p0 = copy.copy(p)
    p0.w2 = np.zeros_like(p.w2)
    g0 = oracle.layer_backward(x, p0, w.offsets, w.timestamps, dy, **kw)
    for k, m in g0["mag"].items():
        if k != "db2":
            assert np.all(m == 0), k
    gz = oracle.layer_backward(x, p, w.offsets, w.timestamps, np.zeros_like(dy), **kw)
    for k, m in gz["mag"].items():
        assert np.all(m == 0), k


# ---------------------------------------------------------------------------
# type-aware rab ("HSTU：Scaling Law 的首次探索" §7.1.4, innovation 2)
# ---------------------------------------------------------------------------

def _typed(lengths, nt, seed, d=8, H=2, nb=32):
    w = _tiny(lengths, d=d, H=H, seed=seed, n_max=max(lengths))
    rng = np.random.default_rng(seed + 1)
    types = rng.integers(0, nt, size=w.total_tokens)
    tb = rng.standard_normal(nt * nt * nb) * 0.5
    w.timestamps = w.timestamps + np.arange(w.total_tokens) ** 3   # many buckets
    return w, types, tb


@pytest.mark.parametrize("nt", [2, 3])
def test_attention_types_bruteforce(nt):
    w, types, tb = _typed([5, 1, 9], nt, seed=40 + nt)
    p = w.layers[0]
    u, v, q, k = _qkv(w)
    got = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, tb, w.num_heads, w.n_max,
                           w.alpha, token_types=types, num_token_types=nt)
    want = _brute_attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, tb, w.num_heads,
                            w.n_max, w.alpha, types=types, nt=nt)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_types_targets_and_cache_bruteforce():
    w = gen.make_ranking(seed=12, users=3, history=[4, 0, 6], candidates=[3, 2, 1],
                         micro_batch=2, d_model=8, num_heads=2, num_layers=1, affine="random",
                         dtype="f32")
    p = w.layers[0]
    rng = np.random.default_rng(5)
    nt = 2
    tb = rng.standard_normal(nt * nt * 32)
    cache = dict(k=rng.standard_normal((w.total_tokens, 8)), v=rng.standard_normal((w.total_tokens, 8)),
                 offsets=w.offsets, timestamps=w.timestamps,
                 types=rng.integers(0, nt, size=w.total_tokens))
    Tc = int(w.cand_offsets[-1])
    cq, ck, cv = (rng.standard_normal((Tc, 8)) for _ in range(3))
    ctypes_ = rng.integers(0, nt, size=Tc)
    m = np.diff(w.cand_offsets)
    got = oracle.attention(cq, ck, cv, w.cand_offsets, w.cand_timestamps, p.pos_bias, tb, 2, w.n_max,
                           num_targets=m, cache=cache, token_types=ctypes_, num_token_types=nt)
    want = _brute_attention(cq, ck, cv, w.cand_offsets, w.cand_timestamps, p.pos_bias, tb, 2, w.n_max,
                            1.0, num_targets=m, cache=cache, types=ctypes_, nt=nt)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_types_single_type_is_the_untyped_rab():
    """Every token of type 0 with the (0, 0) table equal to the untyped one:
    bitwise the untyped result, whatever the other type pairs hold."""
    w, _, _ = _typed([7, 3], 3, seed=50)
    p = w.layers[0]
    u, v, q, k = _qkv(w)
    tb3 = np.random.default_rng(51).standard_normal(9 * 32)
    tb3[:32] = p.time_bias
    got = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, tb3, 2, w.n_max, w.alpha,
                           token_types=np.zeros(w.total_tokens, np.int64), num_token_types=3)
    np.testing.assert_array_equal(got, _attn(w, q, k, v))


def test_attention_types_constant_pair_tables_closed_form():
    """Q = K = 0, no position bias, and each pair's time table a constant
    c[a, b] (asymmetric): AV_i = sum over key types b of
    SiLU(c[type_i, b]) * (prefix sum of v over the keys of type b up to i),
    a per-type np.cumsum. A transposed (key type, query type) lookup fails."""
    nt = 3
    w, types, _ = _typed([11, 6], nt, seed=60)
    p = w.layers[0]
    p.pos_bias[:] = 0.0
    c = np.array([[0.3, -1.2, 2.0], [0.9, 0.1, -0.4], [-2.5, 1.7, 0.6]])
    tb = np.repeat(c.reshape(-1), 32)
    v = np.random.default_rng(61).standard_normal((w.total_tokens, 8))
    z = np.zeros_like(v)
    got = oracle.attention(z, z, v, w.offsets, w.timestamps, p.pos_bias, tb, 2, w.n_max,
                           token_types=types, num_token_types=nt)
    silu = lambda x: x / (1.0 + math.exp(-x))
    for b0 in range(2):
        s, e = int(w.offsets[b0]), int(w.offsets[b0 + 1])
        ty = types[s:e]
        want = np.zeros((e - s, 8))
        for tb_ in range(nt):
            pref = np.cumsum(np.where((ty == tb_)[:, None], v[s:e], 0.0), axis=0)
            want += np.array([silu(c[a, tb_]) for a in ty])[:, None] * pref
        np.testing.assert_allclose(got[s:e], want, rtol=1e-12, atol=1e-13)


def test_attention_types_relabel_equivariance():
    """Renaming the types by a permutation, with the pair tables moved
    accordingly, leaves every output unchanged."""
    nt = 3
    w, types, tb = _typed([8, 5, 2], nt, seed=70)
    p = w.layers[0]
    u, v, q, k = _qkv(w)
    perm = np.array([2, 0, 1])
    tb3 = tb.reshape(nt, nt, 32)
    tb_new = np.empty_like(tb3)
    for a in range(nt):
        for b in range(nt):
            tb_new[perm[a], perm[b]] = tb3[a, b]
    base = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, tb, 2, w.n_max, w.alpha,
                            token_types=types, num_token_types=nt)
    moved = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, tb_new.reshape(-1), 2,
                             w.n_max, w.alpha, token_types=perm[types], num_token_types=nt)
    np.testing.assert_allclose(moved, base, rtol=0, atol=0)
