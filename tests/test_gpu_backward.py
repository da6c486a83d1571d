"""The layer backward pass on the GPU (hstu_layer_bwd, fp32, plain causal
attention) against the oracle's float64 backward, itself pinned by finite
differences of the forward.

Metric, below 1e-4 (the fp32 bound of the forward tests):
* matrices (dX [T, d], dW1 [4d, d], dW2 [d, d]) row by row, as the forward
  tests do: max_t ||g_t - r_t||_inf / max(||r_t||_inf, 1e-6);
* vectors (db1, db2, dgamma, dbeta, the position and time tables' gradients,
  dln1_gamma, dln1_beta) entry by entry: |g_i - r_i| / max(|r_i|, FLOOR *
  max |r|). FLOOR = 1e-2: with the 1e-4 bound an entry is then allowed an
  absolute error of at least 1e-6 max |r|, about 8 fp32 ulps of the tensor's
  largest entry. Entries far below the largest are sums that cancelled down
  to their size, and fp32 accumulation resolves them only to the ulp of the
  terms they cancelled from."""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import f32, i64, row_rel_err, to_np

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-4
FLOOR = 1e-2


def _rel(g, r):
    """Row-normalised for matrices, per entry above the floor for vectors."""
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    assert g.shape == r.shape and np.all(np.isfinite(g))
    if g.size == 0:
        return 0.0
    if g.ndim == 2:
        return row_rel_err(g, r)
    den = np.maximum(np.abs(r), max(FLOOR * np.abs(r).max(), 1e-12))
    return float((np.abs(g - r) / den).max())


@pytest.mark.parametrize("lengths,d,H,alpha,shuffle_ts", [
    ([1, 5, 64, 65, 0, 130], 64, 2, 0.7, False),   # head_dim 32, ragged tails, an empty sequence
    ([200, 3, 64], 128, 2, 1.0, False),            # head_dim 64
    ([100, 33, 257], 512, 8, 1.0, False),          # 8 heads: one 8-wave workgroup per block row
    ([40, 75, 2], 96, 3, 1.0, False),              # 3 heads of 32: a 3-wave workgroup
    ([65, 1, 31], 1024, 16, 0.5, False),           # 16 heads: two head groups per block row
    ([90, 140], 128, 2, 1.0, True),                # timestamps out of order: buckets change often
    ([120, 64, 9], 128, 2, 1.0, "wide"),           # clocks spanning far more than 2^31 units
    (None, None, None, None, False),               # the 1 x 64 fp32 workload
])
def test_layer_backward_matches_oracle(gpu_lib, lengths, d, H, alpha, shuffle_ts):
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    if lengths is None:
        w = gen.make_config(0, affine="random")
    else:
        w = gen.make_custom(lengths, d, H, dtype="f32", seed=61, affine="random")
        w.alpha = alpha
        if shuffle_ts == "wide":
            from tests.test_gpu_time_buckets import _timestamps
            w.timestamps = _timestamps("wide", lengths, np.random.default_rng(64))
            w.layers[0].time_bias = np.random.default_rng(65).standard_normal(32).astype(np.float32)
        elif shuffle_ts:
            rng = np.random.default_rng(63)
            for b in range(len(lengths)):
                s0, s1 = int(w.offsets[b]), int(w.offsets[b + 1])
                w.timestamps[s0:s1] = rng.permutation(w.timestamps[s0:s1])
    d, T = w.d_model, w.total_tokens
    p = w.layers[0]
    dy = np.random.default_rng(62).standard_normal((T, d)).astype(np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    desc = lay.desc
    g = {k: torch.empty(n, dtype=torch.float32, device="cuda") for k, n in [
        ("dw1", 4 * d * d), ("db1", 4 * d), ("dw2", d * d), ("db2", d), ("dgamma", d),
        ("dbeta", d), ("dpos", 2 * w.n_max - 1), ("dtime", w.num_time_buckets)]}
    grads = hstu.make_grads(g["dw1"], g["db1"], g["dw2"], g["db2"], g["dgamma"], g["dbeta"],
                            g["dpos"], g["dtime"])
    dyt = f32(dy)
    dx = torch.empty_like(dyt)
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(desc, dw.jagged))
    hstu.hstu_layer_bwd(desc, lay.params, dw.jagged, dw.x, dyt, dx, grads, ws)
    torch.cuda.synchronize()
    ref = oracle.layer_backward(w.x, p, w.offsets, w.timestamps, dy, w.num_heads, w.n_max,
                                w.alpha, w.ln_eps)
    got = {"dx": to_np(dx), "dw1": to_np(g["dw1"]).reshape(4 * d, d),
           "dw2": to_np(g["dw2"]).reshape(d, d), **{k: to_np(g[k]) for k in
                                                   ("db1", "db2", "dgamma", "dbeta", "dpos", "dtime")}}
    errs = {k: _rel(got[k], ref[k]) for k in got}
    print("backward", lengths, {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL_BWD, (k, e)


def test_layer_backward_empty_batch_zeroes_gradients(gpu_lib):
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu
    desc = hstu.make_desc(64, 2, hstu.HSTU_F32, 15)
    g = [torch.full((n,), 3.0, device="cuda") for n in (4 * 64 * 64, 256, 64 * 64, 64, 64, 64, 15, 32)]
    grads = hstu.make_grads(*g)
    off, ts = i64([0, 0]), i64([0])
    jag = hstu.Jagged(1, 0, 0, hstu.ptr(off), hstu.ptr(ts), None)
    w1 = torch.zeros(256, 64, device="cuda")
    pb, tb = torch.zeros(15, device="cuda"), torch.zeros(32, device="cuda")
    params = hstu.make_params(w1, None, w1[:64], None, None, None, pb, tb)
    hstu.hstu_layer_bwd(desc, params, jag, None, None, None, grads, None)
    torch.cuda.synchronize()
    assert all(float(t.abs().max()) == 0.0 for t in g)


def test_layer_backward_long_sequence_tables_balance(gpu_lib):
    """A sequence longer than the LDS accumulator of position gradients
    (differences up to 16 384): the excess goes to global memory directly.
    Every visible pair adds its score gradient once to the position table and
    once to the time table, so the two tables' sums agree, and the entries
    beyond the accumulator receive their share."""
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    L = 16500
    w = gen.make_custom([L], 32, 1, dtype="f32", seed=71, n_max=L)
    d, T = w.d_model, w.total_tokens
    dy = np.random.default_rng(72).standard_normal((T, d)).astype(np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    g = [torch.empty(n, dtype=torch.float32, device="cuda") for n in
         (4 * d * d, 4 * d, d * d, d, d, d, 2 * w.n_max - 1, w.num_time_buckets)]
    grads = hstu.make_grads(*g)
    dx = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, dw.jagged))
    hstu.hstu_layer_bwd(lay.desc, lay.params, dw.jagged, dw.x, f32(dy), dx, grads, ws)
    torch.cuda.synchronize()
    dpos = to_np(g[6]).astype(np.float64)
    dtime = to_np(g[7]).astype(np.float64)
    assert np.all(np.isfinite(dpos)) and np.all(np.isfinite(dtime))
    center = w.n_max - 1
    # differences below zero are never visible
    assert np.all(dpos[:center] == 0.0)
    scale = np.abs(dpos).sum()
    assert abs(dpos.sum() - dtime.sum()) <= 1e-4 * scale, (dpos.sum(), dtime.sum(), scale)
    # differences 16 384 .. L-1 exist and received gradient
    assert np.count_nonzero(dpos[center + 16384:center + L]) > 0


def test_training_step_in_two_calls(gpu_lib):
    """hstu_layer_fwd_train gives the layer's Y and leaves the activations in
    the workspace; hstu_layer_bwd_after_fwd then gives the gradients of
    hstu_layer_bwd without recomputing the forward."""
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    w = gen.make_custom([300, 7, 129], 256, 4, dtype="f32", seed=81, affine="random")
    d, T = w.d_model, w.total_tokens
    p = w.layers[0]
    dy = np.random.default_rng(82).standard_normal((T, d)).astype(np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, dw.jagged))
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    hstu.hstu_layer_fwd_train(lay.desc, lay.params, dw.jagged, dw.x, y, ws)
    ref_y = oracle.layer(w.x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, w.ln_eps)["y"]
    assert _rel(to_np(y), ref_y) < TOL_BWD
    sizes = [4 * d * d, 4 * d, d * d, d, d, d, 2 * w.n_max - 1, w.num_time_buckets]
    g = [torch.empty(n, dtype=torch.float32, device="cuda") for n in sizes]
    dx = torch.empty((T, d), dtype=torch.float32, device="cuda")
    hstu.hstu_layer_bwd_after_fwd(lay.desc, lay.params, dw.jagged, dw.x, f32(dy), dx, hstu.make_grads(*g), ws)
    torch.cuda.synchronize()
    ref = oracle.layer_backward(w.x, p, w.offsets, w.timestamps, dy, w.num_heads, w.n_max, w.alpha, w.ln_eps)
    names = ["dw1", "db1", "dw2", "db2", "dgamma", "dbeta", "dpos", "dtime"]
    got = {"dx": to_np(dx), **{k: to_np(t) for k, t in zip(names, g)}}
    got["dw1"] = got["dw1"].reshape(4 * d, d)
    got["dw2"] = got["dw2"].reshape(d, d)
    errs = {k: _rel(got[k], ref[k]) for k in got}
    print("two calls", {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL_BWD, (k, e)


def test_layer_backward_over_a_stochastic_length_sample(gpu_lib):
    """Generative training with Stochastic Length ("HSTU：Scaling Law 的首次
    探索" §7.1.5): the sampler's rows of X, dY and the timestamps gathered on
    the device, then the backward over the shorter batch, against the
    oracle's backward over the same sampled sequences."""
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    from tests.helpers import i64
    w = gen.make_custom([400, 40, 520, 0, 260], 128, 2, dtype="f32", seed=85, affine="random", n_max=520)
    d, B, T = w.d_model, w.num_seqs, w.total_tokens
    rng = np.random.default_rng(86)
    off, rows = hstu.hstu_stochastic_length(w.offsets, 1.6, w.n_max, rng.random(B), rng.random(T))
    assert rows.size < T
    n = int(rows.size)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    rows_d, off_d = i64(rows), i64(off)
    dyt = f32(dy)
    xs, dys, dxs = (torch.empty((n, d), dtype=torch.float32, device="cuda") for _ in range(3))
    ts = torch.empty(n, dtype=torch.int64, device="cuda")
    hstu.hstu_gather_rows(n, 4 * d, rows_d, T, dw.x, xs)
    hstu.hstu_gather_rows(n, 4 * d, rows_d, T, dyt, dys)
    hstu.hstu_gather_rows(n, 8, rows_d, T, dw.timestamps, ts)
    jag = hstu.Jagged(B, int(np.diff(off).max()), n, hstu.ptr(off_d), hstu.ptr(ts), None)
    sizes = [4 * d * d, 4 * d, d * d, d, d, d, 2 * w.n_max - 1, w.num_time_buckets]
    g = [torch.empty(k, dtype=torch.float32, device="cuda") for k in sizes]
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, jag))
    hstu.hstu_layer_bwd(lay.desc, lay.params, jag, xs, dys, dxs, hstu.make_grads(*g), ws)
    torch.cuda.synchronize()
    ref = oracle.layer_backward(np.asarray(w.x)[rows], w.layers[0], off, np.asarray(w.timestamps)[rows],
                                dy[rows], w.num_heads, w.n_max, w.alpha, w.ln_eps)
    names = ["dw1", "db1", "dw2", "db2", "dgamma", "dbeta", "dpos", "dtime"]
    got = {"dx": to_np(dxs), **{k: to_np(t) for k, t in zip(names, g)}}
    got["dw1"] = got["dw1"].reshape(4 * d, d)
    got["dw2"] = got["dw2"].reshape(d, d)
    errs = {k: _rel(got[k], ref[k]) for k in got}
    print("stochastic length backward", n, "of", T, {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL_BWD, (k, e)


@pytest.mark.parametrize("two_calls", [False, True])
def test_layer_backward_with_input_norm(gpu_lib, two_calls):
    """With the input LayerNorm before f1 (random gamma1, beta1) the gradient
    reaches X through the residual and through the LayerNorm; dln1_gamma and
    dln1_beta come back too. Both the recomputing call and the two-call
    training step, against the oracle."""
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    w = gen.make_custom([130, 7, 64, 0, 33], 128, 2, dtype="f32", seed=87, affine="random")
    d, T = w.d_model, w.total_tokens
    p = w.layers[0]
    rng = np.random.default_rng(88)
    p.input_norm = True
    p.ln1_gamma = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    p.ln1_beta = (0.2 * rng.standard_normal(d)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    assert lay.desc.input_norm == 1
    sizes = [4 * d * d, 4 * d, d * d, d, d, d, 2 * w.n_max - 1, w.num_time_buckets, d, d]
    g = [torch.empty(k, dtype=torch.float32, device="cuda") for k in sizes]
    grads = hstu.make_grads(*g)
    dx = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, dw.jagged))
    if two_calls:
        y = torch.empty((T, d), dtype=torch.float32, device="cuda")
        hstu.hstu_layer_fwd_train(lay.desc, lay.params, dw.jagged, dw.x, y, ws)
        hstu.hstu_layer_bwd_after_fwd(lay.desc, lay.params, dw.jagged, dw.x, f32(dy), dx, grads, ws)
        ref_y = oracle.layer(w.x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, w.ln_eps)["y"]
        assert _rel(to_np(y), ref_y) < TOL_BWD
    else:
        hstu.hstu_layer_bwd(lay.desc, lay.params, dw.jagged, dw.x, f32(dy), dx, grads, ws)
    torch.cuda.synchronize()
    ref = oracle.layer_backward(w.x, p, w.offsets, w.timestamps, dy, w.num_heads, w.n_max, w.alpha, w.ln_eps)
    names = ["dw1", "db1", "dw2", "db2", "dgamma", "dbeta", "dpos", "dtime", "dln1_gamma", "dln1_beta"]
    got = {"dx": to_np(dx), **{k: to_np(t) for k, t in zip(names, g)}}
    got["dw1"] = got["dw1"].reshape(4 * d, d)
    got["dw2"] = got["dw2"].reshape(d, d)
    errs = {k: _rel(got[k], ref[k]) for k in got}
    print("backward with input norm", two_calls, {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL_BWD, (k, e)
