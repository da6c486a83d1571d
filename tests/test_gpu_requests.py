"""Candidate scoring across two requests of the same users (M-FALCON
caching, "HSTU：Scaling Law 的首次探索" §7.1.5) on the GPU: request 1's
history is cached per layer; request 2 runs only the tokens that arrived
since, against that cache, appends their K/V with hstu_kv_cache_concat, and
scores its candidates against the combined cache. Everything must equal the
oracle's single pass over the whole history."""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import TOL, i64, row_rel_err, to_np

pytestmark = pytest.mark.gpu


def _split_rows(offsets, lens):
    rows = [np.arange(int(offsets[u]), int(offsets[u]) + int(lens[u])) for u in range(len(lens))]
    return np.concatenate(rows) if rows else np.zeros(0, np.int64)


@pytest.mark.parametrize("history,split,cands,b_m", [
    ([150, 70, 1, 0], [100, 20, 1, 0], [6, 0, 65, 3], 4),
    ([64, 130], [64, 65], [1, 129], 128),
])
def test_two_requests_reuse_the_cache(gpu_lib, history, split, cands, b_m):
    import torch
    from hstu_sequential_transducer_jagged_amd import hstu, runner
    w = gen.make_ranking(seed=51, users=len(history), history=history, candidates=cands,
                         micro_batch=b_m, d_model=256, num_heads=4, num_layers=2, affine="random")
    dw = runner.DeviceWorkload(w)
    hl = np.diff(w.offsets)
    l1 = np.asarray(split, np.int64)
    l2 = hl - l1
    r1 = _split_rows(w.offsets, l1)
    r2 = _split_rows(w.offsets + np.concatenate([l1, [0]]), l2)
    o1, o2 = gen.make_jagged(l1), gen.make_jagged(l2)
    off1, off2 = i64(o1), i64(o2)
    ts1, ts2 = i64(np.asarray(w.timestamps)[r1]), i64(np.asarray(w.timestamps)[r2])
    x1 = dw.upload_act(np.asarray(w.x)[r1])
    x2 = dw.upload_act(np.asarray(w.x)[r2])
    jag1 = hstu.Jagged(len(hl), int(l1.max()), int(o1[-1]), hstu.ptr(off1), hstu.ptr(ts1), None)
    jag2 = hstu.Jagged(len(hl), int(l2.max()), int(o2[-1]), hstu.ptr(off2), hstu.ptr(ts2), None)
    L = len(w.layers)
    # request 1: its history alone, K/V kept per layer
    _, k1, v1 = runner.request_forward(dw, jag1, x1)
    c1 = [runner.DeviceCache(off1, ts1, k1[l], v1[l], int(l1.max()), int(o1[-1])) for l in range(L)]
    # request 2: only the new tokens, against request 1's cache
    y2, k2, v2 = runner.request_forward(dw, jag2, x2, [c.c for c in c1])
    c12 = runner.concat_caches(dw, c1, off2, ts2, k2, v2, int(o2[-1]), int(hl.max()))
    plan = runner.RankingPlan(w, b_m)
    cx = dw.upload_act(np.asarray(w.cand_x)[plan.order])
    cts = i64(np.asarray(w.cand_timestamps)[plan.order])
    out = runner.score_candidates(dw, plan, [c.c for c in c12], cx, cts)
    torch.cuda.synchronize()

    # the combined cache is the whole history, user by user
    np.testing.assert_array_equal(c12[0].offsets.cpu().numpy(), w.offsets)
    np.testing.assert_array_equal(c12[0].timestamps.cpu().numpy()[:int(w.offsets[-1])], w.timestamps)
    ref = oracle.ranking(w)
    got = np.zeros((int(w.cand_offsets[-1]), w.d_model))
    got[plan.order] = to_np(out)
    err_c = row_rel_err(got, ref["cand_y"])
    # request 2's history outputs equal the last layer of one pass over the whole history
    full = oracle.stack(w.x, w.layers, w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha,
                        w.ln_eps)
    err_h = row_rel_err(to_np(y2)[:len(r2)], full[r2]) if len(r2) else 0.0
    # layer-0 K of the combined cache equals the projection of the whole history
    k_full = oracle.proj(w.x, w.layers[0].w1, w.layers[0].b1, w.d_model)[3]
    err_k = row_rel_err(to_np(c12[0].k)[:int(w.offsets[-1])], k_full)
    print(f"two requests {history} split {split}: candidates {err_c:.3e}, "
          f"history {err_h:.3e}, cache K {err_k:.3e}")
    assert err_c < TOL["bf16"] and err_h < TOL["bf16"] and err_k < TOL["bf16"]
