"""MI355X (gfx950) HSTU jagged layer forward.

The compute lives in ``libhstu.so`` (hand-written HIP kernels behind the C
ABI of ``include/hstu.h``); ``hstu`` is its ctypes binding and ``runner``
composes the entry points into single layers, stacks and micro-batched
candidate scoring. Importing the package does not load the library.
"""

__all__ = ["hstu", "runner", "build"]
