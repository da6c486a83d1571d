"""Kernel parity on the GPU: each entry point of the C ABI against the CPU
oracle, element by element on the same seeded inputs, at sizes that span
several tiles and ragged tails, plus edge cases."""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import TOL, act_tensor, f32, i32, i64, round_like, row_rel_err, to_np

pytestmark = pytest.mark.gpu

EDGE_LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 0, 200, 31, 33]


def _qkv_inputs(w, dtype):
    """Realistic Q, K, V: the oracle projection of the workload's X, rounded
    the way the device stores them."""
    u, v, q, k = oracle.proj(w.x, w.layers[0].w1, w.layers[0].b1, w.d_model)
    return [round_like(a, dtype) for a in (u, v, q, k)]


def _run_attn(hs, w, dtype, q, k, v, num_targets=None, cache=None, alpha=1.0, no_self=False):
    import torch
    desc = hs.make_desc(w.d_model, w.num_heads, hs.HSTU_BF16 if dtype == "bf16" else hs.HSTU_F32,
                        2 * w.n_max - 1, alpha=alpha, target_no_self=no_self)
    offs, ts = i64(w.offsets), i64(w.timestamps)
    nt = None if num_targets is None else i32(num_targets)
    jag = hs.make_jagged(offs, ts, w.max_seq_len, nt)
    qd, kd, vd = (act_tensor(a, dtype) for a in (q, k, v))
    keep = []
    cch = None
    if cache is not None:
        co, ct = i64(cache["offsets"]), i64(cache["timestamps"])
        ck, cv = act_tensor(cache["k"], dtype), act_tensor(cache["v"], dtype)
        keep = [co, ct, ck, cv]
        cch = hs.make_cache(co, ct, ck, cv, int(np.diff(cache["offsets"]).max()))
    p = w.layers[0]
    pb, tb = f32(p.pos_bias), f32(p.time_bias)
    av = torch.full((max(w.total_tokens, 1), w.d_model), float("nan"), dtype=torch.float32,
                    device="cuda")
    ws = hs.workspace_tensor(hs.hstu_attn_workspace_size(desc, jag))
    hs.hstu_attn_fwd(desc, jag, cch, qd, kd, vd, pb, tb, av, ws)
    torch.cuda.synchronize()
    del keep
    return to_np(av)[:w.total_tokens]


@pytest.mark.parametrize("H", [8, 4, 2, 1, 16, 12, 6])
def test_attn_bf16_edge_lengths(gpu_lib, H):
    w = gen.make_custom(EDGE_LENGTHS, 64 * H, H, dtype="bf16", seed=100 + H, n_max=256)
    u, v, q, k = _qkv_inputs(w, "bf16")
    got = _run_attn(gpu_lib, w, "bf16", q, k, v)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H, w.n_max)
    err = row_rel_err(got, ref)
    print(f"attn bf16 H={H} T={w.total_tokens}: {err:.3e}")
    assert err < TOL["bf16"]


def test_attn_bf16_uneven_work_lists(gpu_lib):
    """Equal-length sequences: the XCD whose cost share holds the cheap early
    tiles gets more items than workgroups, which then take several items."""
    H = 2
    w = gen.make_custom([1024, 1024, 1024, 960], 64 * H, H, dtype="bf16", seed=150, n_max=1024)
    u, v, q, k = _qkv_inputs(w, "bf16")
    got = _run_attn(gpu_lib, w, "bf16", q, k, v)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H, w.n_max)
    err = row_rel_err(got, ref)
    print(f"attn bf16 uneven lists: {err:.3e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("dh,H", [(32, 2), (64, 2), (64, 8), (32, 3), (64, 16), (64, 1)])
def test_attn_f32_edge_lengths(gpu_lib, dh, H):
    w = gen.make_custom(EDGE_LENGTHS, H * dh, H, dtype="f32", seed=200 + dh + H, n_max=256)
    u, v, q, k = _qkv_inputs(w, "f32")
    got = _run_attn(gpu_lib, w, "f32", q, k, v)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H, w.n_max)
    err = row_rel_err(got, ref)
    print(f"attn f32 dh={dh}: {err:.3e}")
    assert err < TOL["f32"]


@pytest.mark.parametrize("dtype,alpha", [("bf16", 0.125), ("bf16", -0.5), ("f32", 0.125)])
def test_attn_alpha(gpu_lib, dtype, alpha):
    H = 4
    dh = 64
    w = gen.make_custom([5, 90, 130], dh * H, H, dtype=dtype, seed=300, n_max=130)
    u, v, q, k = _qkv_inputs(w, dtype)
    got = _run_attn(gpu_lib, w, dtype, q, k, v, alpha=alpha)
    p = w.layers[0]
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H,
                           w.n_max, alpha=alpha)
    assert row_rel_err(got, ref) < TOL[dtype]


@pytest.mark.parametrize("dtype,no_self", [("bf16", False), ("f32", False), ("bf16", True), ("f32", True)])
def test_attn_targets_and_cache(gpu_lib, dtype, no_self):
    """Own tokens = some non-targets then targets, plus a cached history;
    no_self: targets do not see themselves."""
    H = 2
    rng = np.random.default_rng(5)
    w = gen.make_ranking(seed=31, users=5, history=[70, 0, 129, 1, 64],
                         candidates=[40, 3, 65, 0, 130], micro_batch=64, d_model=64 * H,
                         num_heads=H, num_layers=1, dtype=dtype)
    d = w.d_model
    hk = round_like(rng.standard_normal((w.total_tokens, d)) * 0.5, dtype)
    hv = round_like(rng.standard_normal((w.total_tokens, d)) * 0.5, dtype)
    cache = dict(k=hk, v=hv, offsets=w.offsets, timestamps=w.timestamps)
    Tc = int(w.cand_offsets[-1])
    cq, ck, cv = (round_like(rng.standard_normal((Tc, d)) * 0.5, dtype) for _ in range(3))
    m = np.diff(w.cand_offsets).astype(np.int32)
    m = np.maximum(m - np.array([7, 1, 0, 0, 30]), 0).astype(np.int32)  # some non-targets first
    own = gen.Workload(name="own", dtype=dtype, d_model=d, num_heads=H, head_dim=64,
                       n_max=w.n_max + 130, num_time_buckets=32, alpha=1.0, ln_eps=1e-5,
                       offsets=w.cand_offsets, timestamps=w.cand_timestamps, x=None,
                       layers=[gen.make_layer_params(
                           {n: np.random.default_rng(i) for i, n in enumerate(
                               ["w1", "w2", "pos", "time"])}, d, w.n_max + 130, dtype)])
    got = _run_attn(gpu_lib, own, dtype, cq, ck, cv, num_targets=m, cache=cache, no_self=no_self)
    p = own.layers[0]
    ref = oracle.attention(cq, ck, cv, own.offsets, own.timestamps, p.pos_bias, p.time_bias, H,
                           own.n_max, num_targets=m, cache=cache, target_no_self=no_self)
    # a target of a user with no history and no self sees nothing: AV = 0
    empty = np.abs(ref).max(axis=1) == 0
    assert np.all(got[empty] == 0.0)
    err = row_rel_err(got[~empty], ref[~empty])
    print(f"attn {dtype} targets+cache no_self={no_self}: {err:.3e}")
    assert err < TOL[dtype]


def test_attn_long_sequence_sampled_rows(gpu_lib):
    """One 4096-token sequence next to short ones: rows sampled along the
    long sequence, the oracle evaluates only those rows."""
    H = 8
    w = gen.make_custom([4096, 3, 700], 64 * H, H, dtype="bf16", seed=400, n_max=4096)
    u, v, q, k = _qkv_inputs(w, "bf16")
    got = _run_attn(gpu_lib, w, "bf16", q, k, v)
    p = w.layers[0]
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4031, 4095, 4096, 4098, 4099, 4500, 4798])
    ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, H, w.n_max,
                           rows=rows)
    assert row_rel_err(got[rows], ref) < TOL["bf16"]


def test_attn_deterministic(gpu_lib):
    w = gen.make_custom([300, 17, 129], 512, 8, dtype="bf16", seed=500, n_max=300)
    u, v, q, k = _qkv_inputs(w, "bf16")
    a = _run_attn(gpu_lib, w, "bf16", q, k, v)
    b = _run_attn(gpu_lib, w, "bf16", q, k, v)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# projection, norm/gate, output
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,T", [("bf16", 256, 1000), ("bf16", 512, 333), ("bf16", 128, 1),
                                       ("f32", 64, 70), ("f32", 128, 257)])
def test_proj(gpu_lib, dtype, d, T):
    import torch
    hs = gpu_lib
    w = gen.make_custom([T], d, d // 64 if dtype == "bf16" else 2, dtype=dtype, seed=600 + d,
                        affine="random")
    p = w.layers[0]
    desc = hs.make_desc(d, w.num_heads, hs.HSTU_BF16 if dtype == "bf16" else hs.HSTU_F32,
                        2 * w.n_max - 1)
    x, w1, b1 = act_tensor(w.x, dtype), act_tensor(p.w1, dtype), f32(p.b1)
    params = hs.make_params(w1, b1, None, None, None, None, None, None)
    outs = [torch.empty((T, d), dtype=x.dtype, device="cuda") for _ in range(4)]
    hs.hstu_proj_fwd(desc, params, T, x, *outs)
    torch.cuda.synchronize()
    ref = oracle.proj(w.x, p.w1, p.b1, d)
    for name, o, r in zip("UVQK", outs, ref):
        err = row_rel_err(to_np(o), r)
        assert err < (8e-3 if dtype == "bf16" else 1e-5), (name, err)


@pytest.mark.parametrize("dtype,d", [("bf16", 256), ("bf16", 512), ("f32", 64), ("bf16", 1024)])
def test_norm_gate(gpu_lib, dtype, d):
    import torch
    hs = gpu_lib
    T = 517
    rng = np.random.default_rng(d)
    # AV rows with a large common offset (as long causal sums produce)
    av = (rng.standard_normal((T, d)) + 40.0 * rng.standard_normal((T, 1))).astype(np.float32)
    u = round_like(rng.standard_normal((T, d)), dtype)
    gm = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    bt = (0.1 * rng.standard_normal(d)).astype(np.float32)
    desc = hs.make_desc(d, d // 64 if dtype == "bf16" else 2,
                        hs.HSTU_BF16 if dtype == "bf16" else hs.HSTU_F32, 1)
    ud = act_tensor(u, dtype)
    g = torch.empty_like(ud)
    hs.hstu_norm_gate_fwd(desc, T, f32(av), ud, f32(gm), f32(bt), g)
    # in place: g written over u
    hs.hstu_norm_gate_fwd(desc, T, f32(av), ud, f32(gm), f32(bt), ud)
    torch.cuda.synchronize()
    ref = oracle.norm_gate(av, u, gm, bt, 1e-5)
    assert row_rel_err(to_np(g), ref) < (8e-3 if dtype == "bf16" else 1e-5)
    assert torch.equal(g, ud)


@pytest.mark.parametrize("dtype,d,T", [("bf16", 256, 1000), ("bf16", 512, 129), ("f32", 64, 65)])
def test_out(gpu_lib, dtype, d, T):
    import torch
    hs = gpu_lib
    rng = np.random.default_rng(T)
    x = round_like(rng.standard_normal((T, d)), dtype)
    g = round_like(rng.standard_normal((T, d)), dtype)
    w2 = round_like(rng.uniform(-0.1, 0.1, (d, d)), dtype)
    b2 = (0.1 * rng.standard_normal(d)).astype(np.float32)
    desc = hs.make_desc(d, d // 64 if dtype == "bf16" else 2,
                        hs.HSTU_BF16 if dtype == "bf16" else hs.HSTU_F32, 1)
    xd, gd = act_tensor(x, dtype), act_tensor(g, dtype)
    y = torch.empty_like(xd)
    hs.hstu_out_fwd(desc, T, gd, xd, act_tensor(w2, dtype), f32(b2), y)
    torch.cuda.synchronize()
    ref = oracle.output(x, g, w2, b2)
    assert row_rel_err(to_np(y), ref) < (8e-3 if dtype == "bf16" else 1e-5)


def test_embed(gpu_lib):
    import torch
    hs = gpu_lib
    rng = np.random.default_rng(9)
    item = round_like(rng.standard_normal((1000, 512)) * 0.02, "bf16")
    act = round_like(rng.standard_normal((16, 512)) * 0.02, "bf16")
    ids = rng.integers(0, 1000, 777)
    a = rng.integers(0, 16, 777).astype(np.int32)
    ids[5] = 1000   # out of range -> NaN row
    a[9] = -1
    x = torch.empty((777, 512), dtype=torch.bfloat16, device="cuda")
    hs.hstu_embed_fwd(777, 512, hs.HSTU_BF16, act_tensor(item, "bf16"), act_tensor(act, "bf16"),
                      i64(ids), i32(a), x)
    torch.cuda.synchronize()
    got = to_np(x)
    bad = np.zeros(777, bool)
    bad[[5, 9]] = True
    assert np.all(np.isnan(got[bad]))
    ref = oracle.embed(item, act, np.where(bad, 0, ids), np.where(bad, 0, a))
    assert row_rel_err(got[~bad], ref[~bad]) < 4e-3


def test_zero_tokens_and_empty_batch(gpu_lib):
    hs = gpu_lib
    desc = hs.make_desc(512, 8, hs.HSTU_BF16, 255)
    offs = i64([0, 0, 0])
    ts = i64([0])
    jag = hs.make_jagged(offs, ts, 0)
    hs.hstu_attn_fwd(desc, jag, None, None, None, None, None, None, None, None)
    hs.hstu_proj_fwd(desc, hs.make_params(offs, None, None, None, None, None, None, None), 0,
                     None, None, None, None, None)


def test_check_inputs_flags_bad_offsets(gpu_lib):
    hs = gpu_lib
    desc = hs.make_desc(512, 8, hs.HSTU_BF16, 255)
    ts = i64(np.zeros(10))
    good = hs.make_jagged(i64([0, 4, 10]), ts, 6)
    hs.hstu_check_inputs(desc, good)
    for offs, mx in (([0, 5, 4], 6), ([1, 4, 10], 6), ([0, 4, 10], 5)):
        o = i64(offs)
        jag = hs.Jagged(2, mx, 10, hs.ptr(o), hs.ptr(ts), None)
        with pytest.raises(hs.HstuError) as e:
            hs.hstu_check_inputs(desc, jag)
        assert e.value.status == hs.HSTU_E_DATA
    o = i64([0, 4, 10])
    nt = i32([5, 1])
    jag = hs.Jagged(2, 6, 10, hs.ptr(o), hs.ptr(ts), hs.ptr(nt))
    with pytest.raises(hs.HstuError):
        hs.hstu_check_inputs(desc, jag)
