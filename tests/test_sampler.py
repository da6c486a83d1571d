"""The library's Stochastic Length sampler (host code in the C ABI) against
the oracle: bit-exact kept rows and offsets on the same draws (CPU only)."""

import numpy as np
import pytest

import oracle
from hstu_inputs import gen
from hstu_sequential_transducer_jagged_amd import hstu


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(hstu.LIB_PATH):
        from hstu_sequential_transducer_jagged_amd import build
        build.build()
    return hstu.load()


@pytest.mark.parametrize("alpha,n_max,seed", [(1.6, 8192, 0), (1.7, 8192, 1), (2.0, 8192, 2),
                                               (1.5, 16, 3), (1.0, 100, 4), (1.9, 1, 5)])
def test_sampler_matches_oracle(lib, alpha, n_max, seed):
    rng = np.random.default_rng(seed)
    B = 40
    lens = np.minimum(rng.integers(0, 2 * n_max + 2, B), max(n_max, 1))
    lens[:3] = [0, 1, n_max]
    off = gen.make_jagged(lens)
    u = rng.random(B)
    keys = rng.random(int(off[-1]))
    keys[::7] = keys[3] if keys.size > 3 else 0.0          # ties
    got_off, got_rows = hstu.hstu_stochastic_length(off, alpha, n_max, u, keys)
    want_off, want_rows = oracle.stochastic_length(off, alpha, n_max, u, keys)
    np.testing.assert_array_equal(got_off, want_off)
    np.testing.assert_array_equal(got_rows, want_rows)


def test_sampler_workload_sparsity(lib):
    """On 16 sequences of U[2048, 8192] tokens with N = 8192 and alpha = 1.6,
    almost every sequence is cut to floor(8192^0.8) = 1351 tokens."""
    w = gen.make_config(2)
    rng = np.random.default_rng(9)
    off, rows = hstu.hstu_stochastic_length(w.offsets, 1.6, 8192, rng.random(w.num_seqs),
                                            rng.random(w.total_tokens))
    kept = np.diff(off)
    assert set(kept.tolist()) <= set(np.diff(w.offsets).tolist()) | {1351}
    assert (kept == 1351).sum() >= 12
    assert np.all(np.diff(rows[off[0]:off[1]]) > 0)


def test_sampler_validates(lib):
    ok_off = np.array([0, 3], np.int64)
    with pytest.raises(hstu.HstuError):
        hstu.hstu_stochastic_length(ok_off, 2.5, 10, [0.5], np.zeros(3))      # alpha > 2
    with pytest.raises(hstu.HstuError):
        hstu.hstu_stochastic_length(ok_off, 1.6, 0, [0.5], np.zeros(3))       # n_max < 1
    with pytest.raises(hstu.HstuError):
        hstu.hstu_stochastic_length(np.array([0, 3, 2]), 1.6, 10, [0.5, 0.5], np.zeros(3))
    with pytest.raises(hstu.HstuError):
        hstu.hstu_stochastic_length(ok_off, 1.6, 10, [1.5], np.zeros(3))      # u outside [0, 1]
    with pytest.raises(hstu.HstuError):
        hstu.hstu_stochastic_length(ok_off, 1.6, 10, [0.5], np.array([0, np.nan, 1]))
    off, rows = hstu.hstu_stochastic_length(np.zeros(1, np.int64), 1.6, 10, [], [])
    assert off.tolist() == [0] and rows.size == 0
