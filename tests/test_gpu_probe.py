"""The measurement probes on the GPU: the copy is exact and the measured
rates are those of an MI355X-class part (bounds wide enough for any clock
state, tight enough to catch a probe that measures nothing)."""

import pytest

pytestmark = pytest.mark.gpu


def test_probe_copy_is_exact_and_fast(gpu_lib):
    from hstu_sequential_transducer_jagged_amd import probe
    r = probe.copy_hbm(256 << 20, reps=2)
    print(r)
    assert r["copy_exact"]
    assert 500.0 < r["gbs"] < 9000.0


def test_probe_mfma_rate_and_clock(gpu_lib):
    from hstu_sequential_transducer_jagged_amd import probe
    r = probe.mfma_bf16(num_groups=1024, iters=1024, reps=2)
    print(r)
    assert 200.0 < r["tflops"] < 2600.0
    assert 0.3 < r["shader_ghz"] < 3.0
