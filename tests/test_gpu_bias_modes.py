"""The two options of rab on the GPU against the oracle.

* Token types: the type-aware term of "HSTU：Scaling Law 的首次探索" §7.1.4
  (innovation 2), read as one time table per ordered (query type, key type)
  pair beside the shared position table. The tables are drawn N(0, 1) per
  pair and the queries are small, so the bias dominates the scores and a
  lookup in the wrong pair's table moves the output far beyond the
  tolerance (each case also checks that the untyped result is far off).
* The parameter-free bias of "6.2. HSTU的工程突破" eq. 6.2.6,
  -m_p (p_i - p_j) - m_t bucket(t_i - t_j), computed in the kernels
  (HSTU_BIAS_LINEAR), including position differences no table would hold,
  and compared with the table path whose tables hstu_linear_bias_tables
  fills with the same values.

Each runs the bf16 and the fp32 kernels on ragged batches that span several
64-query tiles, plain causal and with targets over a cache, and the whole
layer, fused LayerNorm-gate epilogue included.
"""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import TOL, act_tensor, f32, i32, i64, round_like, row_rel_err, to_np

pytestmark = pytest.mark.gpu

LENGTHS = [300, 1, 64, 65, 130, 0, 33, 257]


def _types(rng, n, nt):
    return rng.integers(0, nt, size=n).astype(np.int32)


def _attn_gpu(hs, dtype, d, H, q, k, v, offsets, ts, pos, tb, n_max, nb, num_targets=None,
              cache=None, types=None, nt=0, linear=None, pos_table_len=None):
    import torch
    desc = hs.make_desc(d, H, hs.HSTU_BF16 if dtype == "bf16" else hs.HSTU_F32,
                        pos_table_len or 2 * n_max - 1, num_time_buckets=nb,
                        num_token_types=nt,
                        bias_mode=hs.HSTU_BIAS_LINEAR if linear else hs.HSTU_BIAS_TABLES,
                        linear_m_p=linear[0] if linear else 0.0,
                        linear_m_t=linear[1] if linear else 0.0)
    keep = []
    offs, tsd = i64(offsets), i64(ts)
    ntd = None if num_targets is None else i32(num_targets)
    tyd = None if types is None else i32(types)
    keep += [offs, tsd, ntd, tyd]
    T = int(offsets[-1])
    jag = hs.make_jagged(offs, tsd, int(np.diff(offsets).max()), ntd, token_types=tyd)
    cch = None
    if cache is not None:
        co, ct = i64(cache["offsets"]), i64(cache["timestamps"])
        ck, cv = act_tensor(cache["k"], dtype), act_tensor(cache["v"], dtype)
        cty = None if cache.get("types") is None else i32(cache["types"])
        keep += [co, ct, ck, cv, cty]
        cch = hs.make_cache(co, ct, ck, cv, int(np.diff(cache["offsets"]).max()), token_types=cty)
    qd, kd, vd = (act_tensor(a, dtype) for a in (q, k, v))
    pb = None if linear else f32(pos)
    tbd = None if linear else f32(tb)
    av = torch.full((max(T, 1), d), float("nan"), dtype=torch.float32, device="cuda")
    ws = hs.workspace_tensor(hs.hstu_attn_workspace_size(desc, jag))
    hs.hstu_check_inputs(desc, jag, cch)
    hs.hstu_attn_fwd(desc, jag, cch, qd, kd, vd, pb, tbd, av, ws)
    torch.cuda.synchronize()
    del keep
    return to_np(av)[:T]


def _qkv(rng, T, d, dtype, q_scale=0.03):
    q = round_like(rng.standard_normal((T, d)) * q_scale, dtype)
    k = round_like(rng.standard_normal((T, d)) * 0.3, dtype)
    v = round_like(rng.standard_normal((T, d)), dtype)
    return q, k, v


def _ts(rng, offsets):
    """Per-sequence increasing clocks with gaps of 2^U s, U ~ U(0, 24): the
    time buckets of a sequence spread over 0..24."""
    out = []
    for b in range(len(offsets) - 1):
        L = int(offsets[b + 1] - offsets[b])
        g = np.floor(2.0 ** rng.uniform(0, 24, size=max(L - 1, 0))).astype(np.int64)
        out.append(1_600_000_000 + np.concatenate([[0], np.cumsum(g)]).astype(np.int64)[:L])
    return np.concatenate(out) if out else np.zeros(0, np.int64)


# ---------------------------------------------------------------------------
# token types
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nt", [2, 3, 4])
def test_typed_attention(gpu_lib, dtype, nt):
    rng = np.random.default_rng(700 + nt)
    H, nb = 2, 32
    d = 64 * H
    offsets = gen.make_jagged(LENGTHS)
    T = int(offsets[-1])
    n_max = max(LENGTHS)
    ts = _ts(rng, offsets)
    q, k, v = _qkv(rng, T, d, dtype)
    pos = (0.1 * rng.standard_normal(2 * n_max - 1)).astype(np.float32)
    tb = rng.standard_normal(nt * nt * nb).astype(np.float32)
    ty = _types(rng, T, nt)
    got = _attn_gpu(gpu_lib, dtype, d, H, q, k, v, offsets, ts, pos, tb, n_max, nb, types=ty, nt=nt)
    ref = oracle.attention(q, k, v, offsets, ts, pos, tb, H, n_max, token_types=ty,
                           num_token_types=nt)
    err = row_rel_err(got, ref)
    plain = oracle.attention(q, k, v, offsets, ts, pos, tb[:nb], H, n_max)
    print(f"{dtype} nt={nt}: err {err:.3e} (untyped reading would be {row_rel_err(got, plain):.2e})")
    assert err < TOL[dtype]
    assert row_rel_err(got, plain) > 0.1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_typed_attention_targets_and_cache(gpu_lib, dtype):
    """Candidates over a typed cached history: the cache rows carry their own
    types, so cache-to-candidate pairs take every (a, b) table."""
    rng = np.random.default_rng(720)
    H, nb, nt = 2, 16, 3
    d = 64 * H
    hist = [70, 0, 129, 1, 64]
    cands = [40, 3, 65, 0, 130]
    c_off = gen.make_jagged(hist)
    offsets = gen.make_jagged(cands)
    Tc, T = int(c_off[-1]), int(offsets[-1])
    hts = _ts(rng, c_off)
    ts = np.empty(T, np.int64)
    for u in range(len(cands)):
        last = hts[c_off[u + 1] - 1] if hist[u] > 0 else 1_600_000_000
        ts[offsets[u]:offsets[u + 1]] = int(last) + int(2 ** rng.uniform(0, 20))
    cache = dict(k=round_like(rng.standard_normal((Tc, d)) * 0.3, dtype),
                 v=round_like(rng.standard_normal((Tc, d)), dtype),
                 offsets=c_off, timestamps=hts, types=_types(rng, Tc, nt))
    q, k, v = _qkv(rng, T, d, dtype)
    m = np.maximum(np.array(cands) - np.array([7, 1, 0, 0, 30]), 0).astype(np.int32)
    n_max = max(hist) + max(cands)
    pos = (0.05 * rng.standard_normal(2 * n_max - 1)).astype(np.float32)
    tb = rng.standard_normal(nt * nt * nb).astype(np.float32)
    ty = _types(rng, T, nt)
    got = _attn_gpu(gpu_lib, dtype, d, H, q, k, v, offsets, ts, pos, tb, n_max, nb, num_targets=m,
                    cache=cache, types=ty, nt=nt)
    ref = oracle.attention(q, k, v, offsets, ts, pos, tb, H, n_max, num_targets=m, cache=cache,
                           token_types=ty, num_token_types=nt)
    empty = np.abs(ref).max(axis=1) == 0
    assert np.all(got[empty] == 0.0)
    err = row_rel_err(got[~empty], ref[~empty])
    print(f"{dtype} typed targets+cache: err {err:.3e}")
    assert err < TOL[dtype]


def _typed_layer(gpu_lib, w, nt, rng):
    from hstu_sequential_transducer_jagged_amd import runner
    import torch
    nb = w.num_time_buckets
    w.layers[0].time_bias = (0.5 * rng.standard_normal(nt * nt * nb)).astype(np.float32)
    ty = _types(rng, w.total_tokens, nt)
    dw = runner.DeviceWorkload(w)
    tyd = i32(ty)
    dw.jagged.token_types = tyd.data_ptr()
    dw.layers[0].desc.num_token_types = nt
    dw.desc.num_token_types = nt
    y = runner.layer_forward(dw, dw.x)
    torch.cuda.synchronize()
    return to_np(y)[:w.total_tokens], ty


@pytest.mark.parametrize("shape", ["split", "fused"])
def test_typed_layer_bf16(gpu_lib, shape):
    """The bf16 layer with token types: a small ragged batch (key ranges split
    over several work items) and 520 short sequences (one head group per row,
    the LayerNorm-gate fused into the attention's epilogue)."""
    rng = np.random.default_rng(740)
    if shape == "split":
        lengths = [300, 64, 3, 200, 129]
    else:
        lengths = list(rng.integers(1, 65, size=520))
    nt = 2
    w = gen.make_custom(lengths, 256, 4, dtype="bf16", seed=741, n_max=max(lengths), affine="random")
    got, ty = _typed_layer(gpu_lib, w, nt, rng)
    p = w.layers[0]
    rows = None if shape == "split" else np.sort(rng.choice(w.total_tokens, 600, replace=False))
    ref = oracle.layer(w.x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, w.ln_eps,
                       rows=rows, token_types=ty, num_token_types=nt)["y"]
    err = row_rel_err(got if rows is None else got[rows], ref)
    print(f"typed bf16 layer ({shape}, T={w.total_tokens}): err {err:.3e}")
    assert err < TOL["bf16"]


# ---------------------------------------------------------------------------
# the parameter-free bias computed in the kernels
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m_p,m_t,nb", [(0.01, 0.3, 32), (0.003, 0.05, 64), (-0.02, 0.7, 8),
                                        (0.0, 0.0, 32)])
def test_linear_attention(gpu_lib, dtype, m_p, m_t, nb):
    """No tables are passed, and the position table length is 1, so the
    position differences (up to 299) lie beyond any table."""
    rng = np.random.default_rng(760 + nb)
    H = 2
    d = 64 * H
    offsets = gen.make_jagged(LENGTHS)
    T = int(offsets[-1])
    n_max = max(LENGTHS)
    ts = _ts(rng, offsets)
    q, k, v = _qkv(rng, T, d, dtype)
    got = _attn_gpu(gpu_lib, dtype, d, H, q, k, v, offsets, ts, None, None, n_max, nb,
                    linear=(m_p, m_t), pos_table_len=1)
    ref = oracle.attention(q, k, v, offsets, ts, None, None, H, n_max, linear_bias=(m_p, m_t),
                           num_time_buckets=nb)
    err = row_rel_err(got, ref)
    print(f"{dtype} linear m_p={m_p} m_t={m_t} nb={nb}: err {err:.3e}")
    assert err < TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_linear_attention_targets_and_cache(gpu_lib, dtype):
    rng = np.random.default_rng(780)
    H, nb = 2, 32
    d = 64 * H
    hist = [70, 0, 129, 1, 64]
    cands = [40, 3, 65, 0, 130]
    c_off = gen.make_jagged(hist)
    offsets = gen.make_jagged(cands)
    Tc, T = int(c_off[-1]), int(offsets[-1])
    hts = _ts(rng, c_off)
    ts = np.empty(T, np.int64)
    for u in range(len(cands)):
        last = hts[c_off[u + 1] - 1] if hist[u] > 0 else 1_600_000_000
        ts[offsets[u]:offsets[u + 1]] = int(last) + int(2 ** rng.uniform(0, 20))
    cache = dict(k=round_like(rng.standard_normal((Tc, d)) * 0.3, dtype),
                 v=round_like(rng.standard_normal((Tc, d)), dtype),
                 offsets=c_off, timestamps=hts)
    q, k, v = _qkv(rng, T, d, dtype)
    m = np.maximum(np.array(cands) - np.array([7, 1, 0, 0, 30]), 0).astype(np.int32)
    n_max = max(hist) + max(cands)
    got = _attn_gpu(gpu_lib, dtype, d, H, q, k, v, offsets, ts, None, None, n_max, nb,
                    num_targets=m, cache=cache, linear=(0.02, 0.4), pos_table_len=1)
    ref = oracle.attention(q, k, v, offsets, ts, None, None, H, n_max, num_targets=m, cache=cache,
                           linear_bias=(0.02, 0.4), num_time_buckets=nb)
    empty = np.abs(ref).max(axis=1) == 0
    assert np.all(got[empty] == 0.0)
    err = row_rel_err(got[~empty], ref[~empty])
    print(f"{dtype} linear targets+cache: err {err:.3e}")
    assert err < TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_linear_matches_filled_tables(gpu_lib, dtype):
    """The in-kernel bias and the table path over hstu_linear_bias_tables
    agree to within the rounding of the bias (one fp32 rounding of each
    product on the table side, a fused log2(e) scale on the kernel side)."""
    import torch
    rng = np.random.default_rng(790)
    H, nb = 2, 32
    d = 64 * H
    offsets = gen.make_jagged(LENGTHS)
    T = int(offsets[-1])
    n_max = max(LENGTHS)
    ts = _ts(rng, offsets)
    q, k, v = _qkv(rng, T, d, dtype)
    m_p, m_t = 0.01, 0.3
    desc = gpu_lib.make_desc(d, H, gpu_lib.HSTU_F32, 2 * n_max - 1, num_time_buckets=nb)
    pos = torch.empty(2 * n_max - 1, dtype=torch.float32, device="cuda")
    tb = torch.empty(nb, dtype=torch.float32, device="cuda")
    gpu_lib.hstu_linear_bias_tables(desc, m_p, m_t, pos, tb)
    torch.cuda.synchronize()
    tab = _attn_gpu(gpu_lib, dtype, d, H, q, k, v, offsets, ts, to_np(pos), to_np(tb), n_max, nb)
    lin = _attn_gpu(gpu_lib, dtype, d, H, q, k, v, offsets, ts, None, None, n_max, nb,
                    linear=(m_p, m_t))
    err = row_rel_err(lin, tab)
    print(f"{dtype} linear vs tables: {err:.3e}")
    assert err < TOL[dtype] / 4


@pytest.mark.parametrize("shape", ["split", "fused"])
def test_linear_layer_bf16(gpu_lib, shape):
    from hstu_sequential_transducer_jagged_amd import runner
    import torch
    rng = np.random.default_rng(800)
    lengths = [300, 64, 3, 200, 129] if shape == "split" else list(rng.integers(1, 65, size=520))
    w = gen.make_custom(lengths, 256, 4, dtype="bf16", seed=801, n_max=max(lengths), affine="random")
    m_p, m_t = 0.004, 0.2
    dw = runner.DeviceWorkload(w)
    L = dw.layers[0]
    L.desc.bias_mode = gpu_lib.HSTU_BIAS_LINEAR
    L.desc.linear_m_p, L.desc.linear_m_t = m_p, m_t
    L.params.pos_bias = None
    L.params.time_bias = None
    y = runner.layer_forward(dw, dw.x)
    torch.cuda.synchronize()
    got = to_np(y)[:w.total_tokens]
    p = w.layers[0]
    p.linear_bias = (m_p, m_t)
    rows = None if shape == "split" else np.sort(rng.choice(w.total_tokens, 600, replace=False))
    ref = oracle.layer(w.x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, w.ln_eps,
                       rows=rows)["y"]
    err = row_rel_err(got if rows is None else got[rows], ref)
    print(f"linear bf16 layer ({shape}, T={w.total_tokens}): err {err:.3e}")
    assert err < TOL["bf16"]
