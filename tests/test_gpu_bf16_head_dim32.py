"""bf16 with head_dim 32 on the GPU against the oracle.

Plain causal batches run on the row-structured bf16 matrix-core kernel
(32-query blocks per head, 16x16x32 bf16 products); targets over a cache,
token types and the parameter-free bias run on the per-row kernel, which
reads the bf16 inputs and computes in fp32. Each case is compared with the
oracle row by row (row-normalised error, the bf16 tolerance) on ragged
batches that span several blocks and end in partial ones, and so is the whole
layer (projection, attention, LayerNorm-gate, output) and the
allocation-free entry point.
"""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import TOL, act_tensor, f32, i64, row_rel_err, to_np
from tests.test_gpu_bias_modes import _attn_gpu as _attn_opts
from tests.test_gpu_bias_modes import _qkv as _qkv_rand
from tests.test_gpu_bias_modes import _ts, _types
from tests.test_gpu_kernels import _qkv_inputs, _run_attn
from tests.test_gpu_time_buckets import _attn_gpu as _attn_tb
from tests.test_gpu_time_buckets import _qkv as _qkv_tb
from tests.test_gpu_time_buckets import _buckets_reached, _timestamps

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 31, 32, 33, 63, 64, 65, 0, 127, 129, 200]
LENGTHS = [300, 1, 64, 65, 130, 0, 33, 257]


@pytest.mark.parametrize("H", [1, 2, 3, 4, 8, 16])
def test_attn_bf16_dh32_edge_lengths(gpu_lib, H):
    w = gen.make_custom(EDGE, 32 * H, H, dtype="bf16", seed=900 + H, n_max=256)
    assert w.d_model // w.num_heads == 32
    u, v, q, k = _qkv_inputs(w, "bf16")
    got = _run_attn(gpu_lib, w, "bf16", q, k, v)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H, w.n_max)
    err = row_rel_err(got, ref)
    print(f"attn bf16 dh32 H={H} T={w.total_tokens}: {err:.3e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("alpha", [0.125, -0.5])
def test_attn_bf16_dh32_alpha(gpu_lib, alpha):
    H = 4
    w = gen.make_custom([5, 90, 130], 32 * H, H, dtype="bf16", seed=910, n_max=130)
    u, v, q, k = _qkv_inputs(w, "bf16")
    got = _run_attn(gpu_lib, w, "bf16", q, k, v, alpha=alpha)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H,
                           w.n_max, alpha=alpha)
    assert row_rel_err(got, ref) < TOL["bf16"]


@pytest.mark.parametrize("kind,nb", [("b32-high", 32), ("b32-mid", 8), ("shuffled", 32),
                                     ("wide", 32), ("huge", 64), ("b32-high", 1)])
def test_attn_bf16_dh32_time_buckets(gpu_lib, kind, nb):
    """Clocks whose blocks fit the 32-bit time path (spans just under 2^31),
    exceed it (spans of years, up to 2^61 units, the 64-bit path), or mix the
    two within one sequence; tables of 1, 8, 32 and 64 buckets."""
    H = 2
    rng = np.random.default_rng(920 + nb)
    w = gen.make_custom(LENGTHS, 32 * H, H, dtype="bf16", seed=920 + nb,
                        n_max=max(LENGTHS))
    w.timestamps = _timestamps(kind, LENGTHS, rng)
    w.num_time_buckets = nb
    w.layers[0].time_bias = rng.standard_normal(nb).astype(np.float32)
    q, k, v = _qkv_tb(w, "bf16")
    got = _attn_tb(gpu_lib, w, "bf16", q, k, v)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H, w.n_max)
    err = row_rel_err(got, ref)
    reached = _buckets_reached(w.timestamps, w.offsets, 64)
    print(f"bf16 dh32 {kind} nb={nb}: buckets {reached[0]}..{reached[-1]}, err {err:.3e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("no_self", [False, True])
def test_attn_bf16_dh32_targets_and_cache(gpu_lib, no_self):
    """Candidates, some non-targets first, over a cached history (the per-row
    kernel on bf16 inputs)."""
    H = 4
    d = 32 * H
    rng = np.random.default_rng(930)
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
    cache = dict(k=_qkv_rand(rng, Tc, d, "bf16")[1], v=_qkv_rand(rng, Tc, d, "bf16")[2],
                 offsets=c_off, timestamps=hts)
    q, k, v = _qkv_rand(rng, T, d, "bf16")
    m = np.maximum(np.array(cands) - np.array([7, 1, 0, 0, 30]), 0).astype(np.int32)
    n_max = max(hist) + max(cands)
    nb = 32
    pos = (0.05 * rng.standard_normal(2 * n_max - 1)).astype(np.float32)
    tb = rng.standard_normal(nb).astype(np.float32)
    own = gen.Workload(name="own", dtype="bf16", d_model=d, num_heads=H, head_dim=32, n_max=n_max,
                       num_time_buckets=nb, alpha=1.0, ln_eps=1e-5, offsets=offsets, timestamps=ts,
                       x=None, layers=[gen.LayerParams(None, None, None, None, None, None, pos, tb)])
    got = _run_attn(gpu_lib, own, "bf16", q, k, v, num_targets=m, cache=cache, no_self=no_self)
    ref = oracle.attention(q, k, v, offsets, ts, pos, tb, H, n_max, num_targets=m, cache=cache,
                           target_no_self=no_self)
    empty = np.abs(ref).max(axis=1) == 0
    assert np.all(got[empty] == 0.0)
    err = row_rel_err(got[~empty], ref[~empty])
    print(f"bf16 dh32 targets+cache no_self={no_self}: err {err:.3e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("nt", [2, 3])
def test_attn_bf16_dh32_typed(gpu_lib, nt):
    rng = np.random.default_rng(940 + nt)
    H, nb = 4, 32
    d = 32 * H
    offsets = gen.make_jagged(LENGTHS)
    T = int(offsets[-1])
    n_max = max(LENGTHS)
    ts = _ts(rng, offsets)
    q, k, v = _qkv_rand(rng, T, d, "bf16")
    pos = (0.1 * rng.standard_normal(2 * n_max - 1)).astype(np.float32)
    tb = rng.standard_normal(nt * nt * nb).astype(np.float32)
    ty = _types(rng, T, nt)
    got = _attn_opts(gpu_lib, "bf16", d, H, q, k, v, offsets, ts, pos, tb, n_max, nb, types=ty, nt=nt)
    ref = oracle.attention(q, k, v, offsets, ts, pos, tb, H, n_max, token_types=ty,
                           num_token_types=nt)
    err = row_rel_err(got, ref)
    print(f"bf16 dh32 typed nt={nt}: err {err:.3e}")
    assert err < TOL["bf16"]
    # the types took effect
    assert row_rel_err(got, oracle.attention(q, k, v, offsets, ts, pos, tb[:nb], H, n_max)) > 0.1


def test_attn_bf16_dh32_linear_bias(gpu_lib):
    """The parameter-free bias computed in the kernel, position differences
    far beyond any table the batch would need."""
    rng = np.random.default_rng(950)
    H, nb = 2, 32
    d = 32 * H
    offsets = gen.make_jagged(LENGTHS)
    T = int(offsets[-1])
    n_max = max(LENGTHS)
    ts = _ts(rng, offsets)
    q, k, v = _qkv_rand(rng, T, d, "bf16")
    mp, mt = 0.0137, 0.21
    got = _attn_opts(gpu_lib, "bf16", d, H, q, k, v, offsets, ts, None, None, n_max, nb,
                     linear=(mp, mt))
    ref = oracle.attention(q, k, v, offsets, ts, None, None, H, n_max, linear_bias=(mp, mt),
                           num_time_buckets=nb)
    err = row_rel_err(got, ref)
    print(f"bf16 dh32 linear bias: err {err:.3e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("lengths,H", [([1, 2, 31, 33, 64, 65, 0, 129], 4), ([300, 77], 8),
                                       ([1] * 9, 2)])
def test_layer_bf16_dh32(gpu_lib, lengths, H):
    """The whole layer: f1 + SiLU split, attention, LayerNorm-gate (a kernel
    of its own: the fused epilogue belongs to the head_dim 64 kernel), f2 +
    residual; no attention workspace."""
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    import torch
    w = gen.make_custom(lengths, 32 * H, H, dtype="bf16", seed=960 + H, n_max=max(lengths),
                        affine="random")
    desc = hstu.make_desc(w.d_model, H, hstu.HSTU_BF16, 2 * w.n_max - 1)
    jag = hstu.make_jagged(i64(w.offsets), i64(w.timestamps), w.max_seq_len)
    assert hstu.hstu_attn_workspace_size(desc, jag) == 0
    dw = runner.DeviceWorkload(w)
    y = runner.layer_forward(dw, dw.x, 0)
    torch.cuda.synchronize()
    got = to_np(y)[:w.total_tokens]
    ref = oracle.layer(w.x, w.layers[0], w.offsets, w.timestamps, H, w.n_max, w.alpha,
                       w.ln_eps)["y"]
    err = row_rel_err(got, ref)
    print(f"layer bf16 dh32 {lengths} H={H}: {err:.3e}")
    assert err < TOL["bf16"]


def test_attn_bf16_dh32_noalloc_matches(gpu_lib):
    """hstu_attn_fwd_noalloc takes the same kernels: bitwise the same AV."""
    from hstu_sequential_transducer_jagged_amd import hstu
    import torch
    H = 4
    w = gen.make_custom([200, 65, 1, 129], 32 * H, H, dtype="bf16", seed=970, n_max=200)
    u, v, q, k = _qkv_inputs(w, "bf16")
    want = _run_attn(gpu_lib, w, "bf16", q, k, v)
    desc = hstu.make_desc(w.d_model, H, hstu.HSTU_BF16, 2 * w.n_max - 1)
    offs, ts = i64(w.offsets), i64(w.timestamps)
    jag = hstu.make_jagged(offs, ts, w.max_seq_len)
    qd, kd, vd = (act_tensor(a, "bf16") for a in (q, k, v))
    p = w.layers[0]
    av = torch.full((w.total_tokens, w.d_model), float("nan"), dtype=torch.float32, device="cuda")
    hstu.hstu_attn_fwd_noalloc(desc, jag, None, qd, kd, vd, f32(p.pos_bias), f32(p.time_bias), av)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(av), want)
