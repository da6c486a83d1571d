"""The layer backward with the attention backward on the bf16 matrix cores
(desc.attn_bwd_bf16 = 1), and with the backward's four products on them as
well (desc.gemm_bwd_bf16 = 1), against the oracle's float64 backward.

Q, K, V and dAV are rounded to bf16 once, P and dS as the operands of their
products, and every sum is fp32. The products dG, dW2, dW1 and dX round
their operands (dY, W2, G, dZ, the input of f1, W1) to bf16 once and sum
in fp32, the weight gradients in fixed splits over the tokens.

Matrices (dX, dW1, dW2) are compared row by row at 2e-2, the bf16 bound of
the forward tests. A vector gradient entry is a sum over tokens or pairs
(db1 over T rows of dZ, a table entry over the dS of every pair at one
position difference or time bucket), so its rounding error scales with the
magnitude of its terms, not with its own size, which cancellation can make
arbitrarily small. The oracle returns that magnitude (``mag``: the sum of
the terms' absolute values, for the table entries one level further down,
into the dot products that make dS). An entry passes when it is within
2e-2 of itself or within 2^-7 of its magnitude. Rounding both operands of
a product to bf16 moves it by at most 2^-8 of its size, so to first order
an entry moves by at most 2^-8 of its magnitude; 2^-7 leaves a factor of
two for the operands' own errors from earlier bf16 steps. A CPU emulation
of these roundings puts the table entries at 0.5e-3 to 1.7e-3 of their
magnitude.
"""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import f32, row_rel_err, to_np

pytestmark = pytest.mark.gpu

TOL = 2e-2
MAG_TOL = 2.0 ** -7


def _rel(g, r, mag=None):
    """Worst error against the bound: row-relative for matrices; for vectors
    per entry, over max(|r|, MAG_TOL/TOL * mag), so that 1.0 * TOL is the
    bound (exactly zero entries with no terms must come back zero)."""
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    assert g.shape == r.shape and np.all(np.isfinite(g))
    if g.size == 0:
        return 0.0
    if g.ndim == 2:
        return row_rel_err(g, r)
    den = np.maximum(np.abs(r), MAG_TOL / TOL * np.asarray(mag, np.float64))
    err = np.abs(g - r)
    assert np.all(err[den == 0] == 0)
    return float((err / np.where(den > 0, den, 1.0)).max())


def _errs(got, ref):
    return {k: _rel(got[k], ref[k], ref["mag"].get(k)) for k in got}


def _grads(d, w):
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu
    g = {k: torch.empty(n, dtype=torch.float32, device="cuda") for k, n in [
        ("dw1", 4 * d * d), ("db1", 4 * d), ("dw2", d * d), ("db2", d), ("dgamma", d),
        ("dbeta", d), ("dpos", 2 * w.n_max - 1), ("dtime", w.num_time_buckets)]}
    return g, hstu.make_grads(g["dw1"], g["db1"], g["dw2"], g["db2"], g["dgamma"], g["dbeta"],
                              g["dpos"], g["dtime"])


def _backward(w, dy, two_calls=False, attn=True, gemm=False):
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    d, T = w.d_model, w.total_tokens
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    desc = hstu.LayerDesc.from_buffer_copy(lay.desc)
    desc.attn_bwd_bf16 = int(attn)
    desc.gemm_bwd_bf16 = int(gemm)
    g, grads = _grads(d, w)
    dyt = f32(dy)
    dx = torch.empty_like(dyt)
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(desc, dw.jagged))
    out = {}
    if two_calls:
        y = torch.empty_like(dyt)
        hstu.hstu_layer_fwd_train(desc, lay.params, dw.jagged, dw.x, y, ws)
        torch.cuda.synchronize()
        out["y"] = to_np(y)
        hstu.hstu_layer_bwd_after_fwd(desc, lay.params, dw.jagged, dw.x, dyt, dx, grads, ws)
    else:
        hstu.hstu_layer_bwd(desc, lay.params, dw.jagged, dw.x, dyt, dx, grads, ws)
    torch.cuda.synchronize()
    return out, {"dx": to_np(dx), "dw1": to_np(g["dw1"]).reshape(4 * d, d),
            "dw2": to_np(g["dw2"]).reshape(d, d),
            **{k: to_np(g[k]) for k in ("db1", "db2", "dgamma", "dbeta", "dpos", "dtime")}}


@pytest.mark.parametrize("lengths,d,H,alpha,ts_kind", [
    ([1, 5, 64, 65, 0, 130], 64, 2, 0.7, None),    # head_dim 32, ragged tails, an empty sequence
    ([200, 3, 64], 128, 2, 1.0, None),             # head_dim 64
    ([100, 33, 257], 512, 8, 1.0, None),           # 8 heads: two 4-wave workgroups per block row
    ([40, 75, 2], 96, 3, 1.0, None),               # 3 heads of 32: a 3-wave workgroup
    ([65, 1, 31], 1024, 16, 0.5, None),            # 16 heads
    ([90, 140], 128, 2, 1.0, "shuffled"),          # timestamps out of order
    ([120, 64, 9], 128, 2, 1.0, "wide"),           # clocks spanning far more than 2^31 units
    ([150, 70], 128, 2, 1.0, "b32-high"),          # spans just under 2^31: buckets to 30 in 32 bits
])
def test_bf16_attention_backward_matches_oracle(gpu_lib, lengths, d, H, alpha, ts_kind):
    w = gen.make_custom(lengths, d, H, dtype="f32", seed=81, affine="random")
    w.alpha = alpha
    if ts_kind in ("wide", "b32-high"):
        from tests.test_gpu_time_buckets import _timestamps
        w.timestamps = _timestamps(ts_kind, lengths, np.random.default_rng(84))
        w.layers[0].time_bias = np.random.default_rng(85).standard_normal(32).astype(np.float32)
    elif ts_kind == "shuffled":
        rng = np.random.default_rng(83)
        for b in range(len(lengths)):
            s0, s1 = int(w.offsets[b]), int(w.offsets[b + 1])
            w.timestamps[s0:s1] = rng.permutation(w.timestamps[s0:s1])
    dy = np.random.default_rng(82).standard_normal((w.total_tokens, w.d_model)).astype(np.float32)
    _, got = _backward(w, dy)
    ref = oracle.layer_backward(w.x, w.layers[0], w.offsets, w.timestamps, dy, w.num_heads, w.n_max,
                                w.alpha, w.ln_eps, magnitudes=True)
    errs = _errs(got, ref)
    print("bf16 backward", lengths, {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL, (k, e)


def test_bf16_backward_in_two_calls(gpu_lib):
    """hstu_layer_fwd_train then hstu_layer_bwd_after_fwd with the flag: dX
    exactly as in one call (no atomics on its path), the gradients that sum
    with fp32 atomics (weights, biases, tables) to their rounding order, and
    everything against the oracle."""
    w = gen.make_custom([150, 7, 64], 128, 2, dtype="f32", seed=86, affine="random")
    dy = np.random.default_rng(87).standard_normal((w.total_tokens, w.d_model)).astype(np.float32)
    _, one = _backward(w, dy)
    fwd, two = _backward(w, dy, two_calls=True)
    ref_y = oracle.layer(w.x, w.layers[0], w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha,
                         w.ln_eps)["y"]
    assert row_rel_err(fwd["y"], ref_y) < TOL
    np.testing.assert_array_equal(one["dx"], two["dx"])
    for k in one:
        scale = np.abs(one[k]).max()
        assert np.abs(two[k] - one[k]).max() <= 1e-5 * scale, k
    ref = oracle.layer_backward(w.x, w.layers[0], w.offsets, w.timestamps, dy, w.num_heads, w.n_max,
                                w.alpha, w.ln_eps, magnitudes=True)
    for k, e in _errs(two, ref).items():
        assert e < TOL, (k, e)


def test_bf16_backward_long_sequence_tables_balance(gpu_lib):
    """A sequence longer than the bf16 kernel's LDS accumulator of position
    gradients (differences up to 8 192): the excess goes to global memory.
    Every visible pair adds its dS once to each table, so the two tables'
    sums agree, and the far entries receive their share."""
    L = 8400
    w = gen.make_custom([L], 64, 1, dtype="f32", seed=88, n_max=L)
    dy = np.random.default_rng(89).standard_normal((w.total_tokens, w.d_model)).astype(np.float32)
    _, got = _backward(w, dy)
    dpos, dtime = got["dpos"].astype(np.float64), got["dtime"].astype(np.float64)
    assert np.all(np.isfinite(dpos)) and np.all(np.isfinite(dtime))
    center = w.n_max - 1
    assert np.all(dpos[:center] == 0.0)
    scale = np.abs(dpos).sum()
    assert abs(dpos.sum() - dtime.sum()) <= 1e-4 * scale, (dpos.sum(), dtime.sum(), scale)
    assert np.count_nonzero(dpos[center + 8192:center + L]) > 0


@pytest.mark.parametrize("lengths,d,H,alpha,ts_kind,attn", [
    ([1, 5, 64, 65, 0, 130], 64, 2, 0.7, None, True),   # head_dim 32, ragged, an empty sequence
    ([100, 33, 257], 512, 8, 1.0, None, True),          # 8 heads, d = 512: 256-row split-K tiles
    ([65, 1, 31], 1024, 16, 0.5, None, True),           # d = 1024
    ([1500, 700, 3], 128, 2, 1.0, None, True),          # T = 2203: 32 splits of 96 tokens, padded
    ([90, 140], 128, 2, 1.0, "shuffled", True),         # timestamps out of order
    ([200, 3, 64], 128, 2, 1.0, None, False),           # the products alone, fp32 attention backward
])
def test_bf16_products_backward_matches_oracle(gpu_lib, lengths, d, H, alpha, ts_kind, attn):
    w = gen.make_custom(lengths, d, H, dtype="f32", seed=91, affine="random")
    w.alpha = alpha
    if ts_kind == "shuffled":
        rng = np.random.default_rng(92)
        for b in range(len(lengths)):
            s0, s1 = int(w.offsets[b]), int(w.offsets[b + 1])
            w.timestamps[s0:s1] = rng.permutation(w.timestamps[s0:s1])
    dy = np.random.default_rng(93).standard_normal((w.total_tokens, w.d_model)).astype(np.float32)
    _, got = _backward(w, dy, attn=attn, gemm=True)
    ref = oracle.layer_backward(w.x, w.layers[0], w.offsets, w.timestamps, dy, w.num_heads, w.n_max,
                                w.alpha, w.ln_eps, magnitudes=True)
    errs = _errs(got, ref)
    print("bf16 products backward", lengths, attn, {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL, (k, e)


@pytest.mark.parametrize("two_calls,attn", [(False, True), (True, True), (False, False)])
def test_bf16_products_backward_with_input_norm(gpu_lib, two_calls, attn):
    """With the input LayerNorm, dW1 contracts dZ with the normalised input
    and dX comes back through the LayerNorm: the bf16 products (fp32
    attention backward) against the oracle, in one call and in the two-call
    step, with the attention on bf16 as well or not. The two-call dX equals
    the one-call dX exactly (fixed splits, no atomics on its path)."""
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    w = gen.make_custom([130, 7, 64, 0, 33], 128, 2, dtype="f32", seed=94, affine="random")
    d, T = w.d_model, w.total_tokens
    p = w.layers[0]
    rng = np.random.default_rng(95)
    p.input_norm = True
    p.ln1_gamma = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    p.ln1_beta = (0.2 * rng.standard_normal(d)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    desc = hstu.LayerDesc.from_buffer_copy(lay.desc)
    desc.attn_bwd_bf16 = int(attn)
    desc.gemm_bwd_bf16 = 1
    sizes = [4 * d * d, 4 * d, d * d, d, d, d, 2 * w.n_max - 1, w.num_time_buckets, d, d]
    g = [torch.empty(k, dtype=torch.float32, device="cuda") for k in sizes]
    grads = hstu.make_grads(*g)
    dx = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(desc, dw.jagged))
    hstu.hstu_layer_bwd(desc, lay.params, dw.jagged, dw.x, f32(dy), dx, grads, ws)
    torch.cuda.synchronize()
    dx_one = to_np(dx)
    if two_calls:
        y = torch.empty((T, d), dtype=torch.float32, device="cuda")
        hstu.hstu_layer_fwd_train(desc, lay.params, dw.jagged, dw.x, y, ws)
        hstu.hstu_layer_bwd_after_fwd(desc, lay.params, dw.jagged, dw.x, f32(dy), dx, grads, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(dx), dx_one)
        # y of the forward call (f1 and f2 on bf16)
        ref_y = oracle.layer(w.x, p, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha, w.ln_eps)["y"]
        assert row_rel_err(to_np(y), ref_y) < TOL
    ref = oracle.layer_backward(w.x, p, w.offsets, w.timestamps, dy, w.num_heads, w.n_max, w.alpha, w.ln_eps,
                                magnitudes=True)
    names = ["dw1", "db1", "dw2", "db2", "dgamma", "dbeta", "dpos", "dtime", "dln1_gamma", "dln1_beta"]
    got = {"dx": to_np(dx), **{k: to_np(t) for k, t in zip(names, g)}}
    got["dw1"] = got["dw1"].reshape(4 * d, d)
    got["dw2"] = got["dw2"].reshape(d, d)
    errs = _errs(got, ref)
    print("bf16 products backward with input norm", two_calls, attn, {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e < TOL, (k, e)


def test_bf16_products_weight_gradients_deterministic(gpu_lib):
    """The split weight gradients are summed in a fixed order: two calls give
    bit-identical dW1 and dW2."""
    w = gen.make_custom([700, 300], 128, 2, dtype="f32", seed=96, affine="random")
    dy = np.random.default_rng(97).standard_normal((w.total_tokens, w.d_model)).astype(np.float32)
    _, a = _backward(w, dy, gemm=True)
    _, b = _backward(w, dy, gemm=True)
    for k in ("dw1", "dw2", "dx"):
        np.testing.assert_array_equal(a[k], b[k])
