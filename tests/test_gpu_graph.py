"""HIP graphs of the library's calls (runner.capture): each replay, with
eager work and synchronisations between replays, gives bitwise the eager
result."""

import numpy as np
import pytest

from hstu_inputs import gen

pytestmark = pytest.mark.gpu


def _replays_match(eager_fn, graphed, out, n=3):
    import torch
    ref = eager_fn().clone()
    for i in range(n):
        graphed.replay()
        other = eager_fn()          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs"
        assert torch.equal(other, ref)


@pytest.mark.parametrize("dtype,lengths,d,H", [("f32", [64], 64, 2), ("bf16", [3, 130, 64, 0, 257], 256, 4),
                                               ("f32", [300, 17], 256, 4)])
def test_layer_graph_replays_match_eager(gpu_lib, dtype, lengths, d, H):
    import torch
    from hstu_sequential_transducer_jagged_amd import runner
    w = gen.make_custom(lengths, d, H, dtype=dtype, seed=91, affine="random")
    dw = runner.DeviceWorkload(w)
    eager = lambda: runner.layer_forward(dw, dw.x, 0)
    g, y = runner.capture(runner.layer_forward, dw, dw.x, 0)
    _replays_match(eager, g, y)


def test_stack_graph_replays_match_eager(gpu_lib):
    from hstu_sequential_transducer_jagged_amd import runner
    w = gen.make_custom([40, 1, 200, 77], 128, 2, dtype="bf16", seed=92, num_layers=3, affine="random")
    dw = runner.DeviceWorkload(w)
    eager = lambda: runner.stack_forward(dw)
    g, h = runner.capture(runner.stack_forward, dw)
    _replays_match(eager, g, h)
