"""hstu_attn_fwd_noalloc (the attention without a workspace argument, its
work list and partial outputs in a static device array) against
hstu_attn_fwd with a caller workspace, through the C ABI, on two calls in a
row: the second smaller than the first, so that it runs over what the first
left in the array. Where the key-range splits are the same the two entry
points run the same kernels on the same plan and agree bitwise; where the
static array caps the splits, the partial sums are grouped differently and
the results agree to the bf16 tolerance (and both match the oracle)."""

import ctypes

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import TOL, act_tensor, f32, i64, round_like, row_rel_err, to_np

pytestmark = pytest.mark.gpu


def _inputs(lengths, H, seed):
    w = gen.make_custom(lengths, 64 * H, H, dtype="bf16", seed=seed, n_max=max(lengths))
    rng = np.random.default_rng(seed)
    T, d = w.total_tokens, w.d_model
    q = round_like(rng.uniform(-0.1, 0.5, (T, d)), "bf16")
    k = round_like(rng.uniform(-0.1, 0.5, (T, d)), "bf16")
    v = round_like(rng.standard_normal((T, d)) * 0.5, "bf16")
    return w, q, k, v


def _both(hs, w, q, k, v):
    import torch
    desc = hs.make_desc(w.d_model, w.num_heads, hs.HSTU_BF16, 2 * w.n_max - 1)
    offs, ts = i64(w.offsets), i64(w.timestamps)
    jag = hs.make_jagged(offs, ts, w.max_seq_len)
    qd, kd, vd = (act_tensor(a, "bf16") for a in (q, k, v))
    p = w.layers[0]
    pb, tb = f32(p.pos_bias), f32(p.time_bias)
    T, d = w.total_tokens, w.d_model
    av_ws = torch.full((T, d), float("nan"), device="cuda")
    av_st = torch.full((T, d), float("nan"), device="cuda")
    ws = hs.workspace_tensor(hs.hstu_attn_workspace_size(desc, jag))
    hs.hstu_attn_fwd(desc, jag, None, qd, kd, vd, pb, tb, av_ws, ws)
    lib = hs.load()
    P = ctypes.c_void_p
    st = lib.hstu_attn_fwd_noalloc(ctypes.byref(desc), ctypes.byref(jag), None, P(qd.data_ptr()),
                                   P(kd.data_ptr()), P(vd.data_ptr()), P(pb.data_ptr()), P(tb.data_ptr()),
                                   P(av_st.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    assert st == hs.HSTU_OK, lib.hstu_last_error()
    torch.cuda.synchronize()
    return to_np(av_ws), to_np(av_st)


def test_noalloc_matches_the_workspace_entry_point(gpu_lib):
    # call 1: 2 x 4096 tokens, d 512: 128 query tiles -> 4 key-range splits
    # in hstu_attn_fwd (63 MiB of partial outputs), capped to 2 by the 32 MiB
    # array; call 2: smaller, 1024 + 300 tokens, d 256: 21 tiles -> 8 splits
    # (10 MiB), the same plan in both entry points
    for lengths, H, seed, same_plan in (([4096, 4000], 8, 901, False), ([1024, 300], 4, 902, True)):
        w, q, k, v = _inputs(lengths, H, seed)
        got_ws, got_st = _both(gpu_lib, w, q, k, v)
        assert np.all(np.isfinite(got_st))
        if same_plan:
            assert np.array_equal(got_ws, got_st)
        else:
            assert row_rel_err(got_st, got_ws) < TOL["bf16"]
        p = w.layers[0]
        o = w.offsets
        rows = np.array([0, 1, 500, int(o[1]) - 1, int(o[1]), int(o[2]) - 1])
        ref = oracle.attention(q, k, v, w.offsets, w.timestamps, p.pos_bias, p.time_bias, w.num_heads,
                               w.n_max, rows=rows)
        err = row_rel_err(got_st[rows], ref)
        print(f"noalloc {lengths} H={H}: vs oracle {err:.3e}, vs workspace entry point "
              f"{row_rel_err(got_st, got_ws):.3e}")
        assert err < TOL["bf16"]
