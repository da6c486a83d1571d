"""ctypes binding of the measurement probes (``libhstu_probe.so``,
``include/hstu_probe.h``): the bf16 matrix-core rate with no memory
traffic, a streaming HBM copy, and the shader clock under matrix-core load.
The benchmark reports them beside the published peaks; they are not part of
the layer. Each function times its launch with HIP events on the current
torch stream."""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu_probe.so")
EXPORTS = ("hstu_probe_mfma_bf16", "hstu_probe_copy")
MFMA_THREADS = 256
FLOP_PER_ROUND = 4 * 32 * 32 * 16 * 2     # four 32x32x16 MFMAs per wave per round

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build the HIP libraries first "
                           "(python -m hstu_sequential_transducer_jagged_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.hstu_probe_mfma_bf16.restype = ctypes.c_int
    lib.hstu_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P]
    lib.hstu_probe_copy.restype = ctypes.c_int
    lib.hstu_probe_copy.argtypes = [P, P, ctypes.c_size_t, P]
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


def mfma_bf16(num_groups: int = 2048, iters: int = 4096, reps: int = 3) -> dict:
    """Best of `reps` launches: TFLOP/s of the MFMA loop and the shader clock
    (GHz, median over workgroups of s_memtime / s_memrealtime ticks)."""
    import torch
    lib = load()
    s = torch.cuda.current_stream()
    sink = torch.zeros(MFMA_THREADS, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * num_groups, dtype=torch.int64, device="cuda")
    flop = float(num_groups) * 4 * iters * FLOP_PER_ROUND
    best, ghz = 0.0, 0.0
    for _ in range(reps + 1):            # the first launch warms up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        _check(lib.hstu_probe_mfma_bf16(num_groups, iters, sink.data_ptr(), clocks.data_ptr(),
                                        s.cuda_stream), "hstu_probe_mfma_bf16")
        e1.record(s)
        torch.cuda.synchronize()
        tflops = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
        c = clocks.view(-1, 2).double()
        g = float((0.1 * c[:, 0] / c[:, 1].clamp(min=1)).median())
        if tflops > best:
            best, ghz = tflops, g
    return {"tflops": best, "shader_ghz": ghz, "groups": num_groups, "iters": iters}


def copy_hbm(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """Best of `reps` copies of nbytes: GB/s counting bytes read plus written."""
    import torch
    lib = load()
    s = torch.cuda.current_stream()
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = 0.0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        _check(lib.hstu_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, s.cuda_stream),
               "hstu_probe_copy")
        e1.record(s)
        torch.cuda.synchronize()
        best = max(best, 2.0 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    ok = bool(torch.equal(src, dst))
    del src, dst
    return {"gbs": best, "bytes": nbytes, "copy_exact": ok}
