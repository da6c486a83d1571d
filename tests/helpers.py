"""Shared helpers for the GPU parity tests: device upload of test inputs and
the error metric.

Error metric (row-normalised max relative error): for an output tensor
with rows t, max_t ||g_t - r_t||_inf / max(||r_t||_inf, 1e-6). The bf16
tolerance is 2e-2 and the fp32 one 1e-4.
"""

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}


def row_rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-6)
    return float((num / den).max())


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def act_tensor(a, dtype, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def round_like(a, dtype):
    """Values as the device holds them (bf16 rounding for bf16)."""
    from hstu_inputs.gen import bf16_round
    a = np.asarray(a, np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def i64(a, device="cuda"):
    import torch
    return torch.from_numpy(np.asarray(a, np.int64)).to(device)


def i32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.asarray(a, np.int32)).to(device)


def f32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def oracle_pool_map(fn, args, workers=8):
    """fn(*a) for each a in args, in a pool of CPU worker processes (spawned,
    so they never inherit a GPU context; they run the float64 oracle only).
    Results come back in the order of args."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import os
    n = max(1, min(workers, len(args), os.cpu_count() or 1))
    if n == 1:
        return [fn(*a) for a in args]
    with cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                initializer=_one_blas_thread) as ex:
        return list(ex.map(fn, *zip(*args)))


def _one_blas_thread():
    """Pool workers keep to one BLAS thread each: the pool supplies the
    parallelism, and nested thread pools would oversubscribe the cores."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
