"""Layer, stack and ranking parity on the GPU against the CPU oracle, on the
five workloads (full-size ones checked on sampled rows, sequences or users
the oracle can evaluate in seconds)."""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from tests.helpers import TOL, oracle_pool_map, row_rel_err, to_np

pytestmark = pytest.mark.gpu


def _runner():
    from hstu_sequential_transducer_jagged_amd import runner
    return runner


def _sync():
    import torch
    torch.cuda.synchronize()


def _layer_gpu(w, l=0, k_out=False):
    runner = _runner()
    dw = runner.DeviceWorkload(w)
    if not k_out:
        y = runner.layer_forward(dw, dw.x, l)
        _sync()
        return to_np(y)[:w.total_tokens]
    kk, vv = dw.empty_act(w.total_tokens), dw.empty_act(w.total_tokens)
    y = runner.layer_forward(dw, dw.x, l, k_out=kk, v_out=vv)
    _sync()
    return to_np(y)[:w.total_tokens], to_np(kk), to_np(vv)


def _oracle_layer(w, l=0, rows=None, x=None):
    x = w.x if x is None else x
    return oracle.layer(x, w.layers[l], w.offsets, w.timestamps, w.num_heads, w.n_max, w.alpha,
                        w.ln_eps, rows=rows)


@pytest.mark.parametrize("affine", ["default", "random"])
def test_config0_fp32_layer(gpu_lib, affine):
    w = gen.make_config(0, affine=affine)
    got = _layer_gpu(w)
    err = row_rel_err(got, _oracle_layer(w)["y"])
    print(f"config 0 ({affine}): {err:.3e}")
    assert err < TOL["f32"]


@pytest.mark.parametrize("affine", ["default", "random"])
def test_config1_bf16_layer_full(gpu_lib, affine):
    w = gen.make_config(1, affine=affine)
    got = _layer_gpu(w)
    err = row_rel_err(got, _oracle_layer(w)["y"])
    print(f"config 1 ({affine}) T={w.total_tokens}: {err:.3e}")
    assert err < TOL["bf16"]


def test_config2_bf16_layer_sampled_rows(gpu_lib):
    """Full-size workload 2 (16 sequences up to 8192), in the launch the
    benchmark times; the oracle evaluates 16 rows of every sequence: its
    first and last rows and 14 drawn between them."""
    w = gen.make_config(2)
    got = _layer_gpu(w)
    o = w.offsets
    rng = np.random.default_rng(2)
    rows = np.concatenate([np.unique(np.concatenate([[o[b], o[b + 1] - 1],
                                                     rng.integers(o[b], o[b + 1], 14)]))
                           for b in range(w.num_seqs)])
    ref = _oracle_layer(w, rows=rows)["y"]
    per_seq = [row_rel_err(got[rows[(rows >= o[b]) & (rows < o[b + 1])]],
                           ref[(rows >= o[b]) & (rows < o[b + 1])]) for b in range(w.num_seqs)]
    worst = int(np.argmax(per_seq))
    print(f"config 2: {rows.size} rows over {w.num_seqs} sequences; worst sequence {worst} "
          f"(length {int(w.lengths[worst])}) {per_seq[worst]:.3e}")
    assert max(per_seq) < TOL["bf16"]


@pytest.mark.parametrize("lengths,H", [([1, 2, 63, 64, 65, 0, 129], 4), ([128] * 5, 8),
                                       ([1] * 9, 2), ([300], 1)])
def test_small_bf16_layers(gpu_lib, lengths, H):
    w = gen.make_custom(lengths, 64 * H, H, dtype="bf16", seed=sum(lengths) + H,
                        n_max=max(lengths), affine="random")
    got = _layer_gpu(w)
    assert row_rel_err(got, _oracle_layer(w)["y"]) < TOL["bf16"]


def test_k_out_v_out_match_projection(gpu_lib):
    w = gen.make_custom([50, 7], 256, 4, dtype="bf16", seed=77, n_max=50)
    y, kk, vv = _layer_gpu(w, k_out=True)
    r = _oracle_layer(w)
    assert row_rel_err(kk[:57], r["k"]) < 8e-3
    assert row_rel_err(vv[:57], r["v"]) < 8e-3
    assert row_rel_err(y, r["y"]) < TOL["bf16"]


# ---------------------------------------------------------------------------
# workload 3: 8-layer stack over item + action embeddings
# ---------------------------------------------------------------------------

def _sub_workload(w, seqs):
    """The chosen sequences of a workload as a workload of their own
    (sequences are independent in the forward)."""
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    sub = gen.Workload(**{f: getattr(w, f) for f in gen.Workload.__dataclass_fields__})
    sub.offsets = gen.make_jagged([int(w.offsets[b + 1] - w.offsets[b]) for b in seqs])
    sub.timestamps = w.timestamps[rows]
    if w.x is not None:
        sub.x = w.x[rows]
    if w.item_ids is not None:
        sub.item_ids = w.item_ids[rows]
        sub.actions = w.actions[rows]
    return sub, rows


@pytest.fixture(scope="module")
def config3_run(gpu_lib):
    runner = _runner()
    w = gen.make_config(3)
    dw = runner.DeviceWorkload(w)
    outs = runner.stack_forward(dw, return_all=True)
    _sync()
    return w, [to_np(o)[:w.total_tokens] for o in outs]


def test_config3_embedding(config3_run):
    w, outs = config3_run
    rows = np.arange(0, w.total_tokens, 997)
    ref = oracle.embed(w.item_emb, w.action_emb, w.item_ids[rows], w.actions[rows])
    assert row_rel_err(outs[0][rows], ref) < 4e-3


def _oracle_stack_one(x0, layers, offsets, timestamps, num_heads, n_max, alpha, eps):
    return oracle.stack(x0, layers, offsets, timestamps, num_heads, n_max, alpha, eps)


def test_config3_stack_end_to_end(config3_run):
    """Whole 8-layer stack on 16 sequences spread over the length
    distribution (one per quantile of the distinct lengths, from 32 to the
    longest), each recomputed by the oracle from its embeddings."""
    w, outs = config3_run
    L = w.lengths
    uniq = np.unique(L)
    picks = uniq[np.unique(np.round(np.linspace(0, uniq.size - 1, 16)).astype(int))]
    seqs = [int(np.nonzero(L == l)[0][0]) for l in picks]
    jobs = []
    for b in seqs:
        sub, _ = _sub_workload(w, [b])
        x0 = oracle.embed(w.item_emb, w.action_emb, sub.item_ids, sub.actions)
        jobs.append((x0, w.layers, sub.offsets, sub.timestamps, w.num_heads, w.n_max, w.alpha,
                     w.ln_eps))
    refs = oracle_pool_map(_oracle_stack_one, jobs)
    errs = []
    for b, ref in zip(seqs, refs):
        rows = np.arange(w.offsets[b], w.offsets[b + 1])
        errs.append(row_rel_err(outs[-1][rows], ref))
    worst = int(np.argmax(errs))
    print(f"config 3 end-to-end over {len(seqs)} sequences (lengths {[int(L[b]) for b in seqs]}); "
          f"worst: length {int(L[seqs[worst]])} {errs[worst]:.3e}")
    assert max(errs) < TOL["bf16"]


def test_config3_teacher_forced_layers(config3_run):
    """Each layer fed the device's own bf16 input: separates the per-layer
    kernel error from error carried through the stack."""
    w, outs = config3_run
    rng = np.random.default_rng(3)
    L = w.lengths
    long_seq = int(np.argmax(L))
    rows = np.concatenate([rng.choice(w.total_tokens, 24, replace=False),
                           [int(w.offsets[long_seq + 1]) - 1]])
    rows.sort()
    for l in range(len(w.layers)):
        ref = _oracle_layer(w, l, rows=rows, x=outs[l])["y"]
        err = row_rel_err(outs[l + 1][rows], ref)
        print(f"config 3 layer {l} teacher-forced: {err:.3e}")
        assert err < TOL["bf16"]


# ---------------------------------------------------------------------------
# workload 4: micro-batched candidate scoring over a cached history
# ---------------------------------------------------------------------------

def _ranking_gpu(w, b_m=None):
    runner = _runner()
    dw = runner.DeviceWorkload(w)
    plan = runner.RankingPlan(w, b_m)
    out = to_np(runner.ranking_forward(dw, plan))
    res = np.zeros_like(out)
    res[plan.order] = out
    return res


def _sub_ranking(w, users):
    hist_rows = np.concatenate([np.arange(w.offsets[u], w.offsets[u + 1]) for u in users])
    cand_rows = np.concatenate([np.arange(w.cand_offsets[u], w.cand_offsets[u + 1]) for u in users])
    sub = gen.Workload(**{f: getattr(w, f) for f in gen.Workload.__dataclass_fields__})
    sub.offsets = gen.make_jagged([int(w.offsets[u + 1] - w.offsets[u]) for u in users])
    sub.cand_offsets = gen.make_jagged([int(w.cand_offsets[u + 1] - w.cand_offsets[u]) for u in users])
    sub.x, sub.timestamps = w.x[hist_rows], w.timestamps[hist_rows]
    sub.cand_x, sub.cand_timestamps = w.cand_x[cand_rows], w.cand_timestamps[cand_rows]
    return sub, cand_rows


@pytest.mark.parametrize("b_m", [1, 2, 5, 128])
def test_small_ranking_full(gpu_lib, b_m):
    w = gen.make_ranking(seed=41, users=4, history=[100, 0, 65, 1], candidates=[9, 4, 0, 130],
                         micro_batch=b_m, d_model=256, num_heads=4, num_layers=2,
                         affine="random")
    got = _ranking_gpu(w)
    ref = oracle.ranking(w)["cand_y"]
    err = row_rel_err(got, ref)
    print(f"small ranking b_m={b_m}: {err:.3e}")
    assert err < TOL["bf16"]


def test_ranking_batched_equals_independent(gpu_lib):
    """Candidates scored in micro-batches against the cache equal each
    candidate scored alone after its user's history (oracle)."""
    w = gen.make_ranking(seed=43, users=2, history=[70, 129], candidates=[5, 3], micro_batch=2,
                         d_model=256, num_heads=4, num_layers=2)
    got = _ranking_gpu(w)
    for u in range(2):
        for c in range(int(w.cand_offsets[u + 1] - w.cand_offsets[u])):
            ref = oracle.ranking_independent(w, u, c)
            err = row_rel_err(got[w.cand_offsets[u] + c][None], ref[None])
            assert err < TOL["bf16"], (u, c, err)


def _oracle_ranking(sub):
    return oracle.ranking(sub)["cand_y"]


def test_config4_ranking_sampled_users(gpu_lib):
    """Workload 4 at full size on the device; the oracle rescoring 8 of the
    32 users (every fourth, each with its 4096-token history and 512
    candidates through 4 layers)."""
    w = gen.make_config(4)
    got = _ranking_gpu(w)
    users = list(range(0, 32, 4))
    refs = oracle_pool_map(_oracle_ranking, [(_sub_ranking(w, [u])[0],) for u in users])
    errs = []
    for u, ref in zip(users, refs):
        rows = np.arange(w.cand_offsets[u], w.cand_offsets[u + 1])
        errs.append(row_rel_err(got[rows], ref))
    worst = int(np.argmax(errs))
    print(f"config 4 users {users}: worst user {users[worst]} {errs[worst]:.3e}")
    assert max(errs) < TOL["bf16"]
