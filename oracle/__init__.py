"""CPU oracle for the HSTU jagged layer forward (test infrastructure).

Plain, slow, float64 NumPy evaluation of the layer's defining equations. It
exists to check the HIP path and is used only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The product path never imports it, and it shares no code with the HIP
library.
"""

from .hstu_oracle import (  # noqa: F401
    attention,
    embed,
    genrank_bias,
    layer,
    layer_backward,
    layernorm,
    norm_gate,
    output,
    proj,
    ranking,
    ranking_independent,
    silu,
    silu_grad,
    silu_grad2,
    stack,
    stochastic_length,
    time_bucket,
)
