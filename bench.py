#!/usr/bin/env python3
"""Benchmark: one HSTU layer forward on the long jagged bf16 workload.

Workload (default ``--workload 2``): 16 sequences with lengths uniform on
[2048, 8192] (the first fixed at 8192), d_model 512, 8 heads of 64, bf16,
seeded synthetic inputs (no dataset exists for it; see hstu_inputs.gen).

A step is one pass of the whole layer path: projection (f1 + SiLU + split),
jagged causal SiLU attention with the position/time bias, LayerNorm-gate and
f2 + residual, each launched through its C-ABI entry point on one stream,
inputs resident in HBM. Steps are timed with HIP events; the attention
kernel's own launches are bracketed by events inside the same timed region.

Prints ONE JSON line (rank 0, one GPU). Only N = 1 is supported.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "HSTU layer fwd tokens/s; jagged attn TFLOP/s and % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate CPU seconds for the oracle sample")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run a plain elementwise copy of known size (512 MiB read, "
                         "512 MiB written) so that HBM counters can be scaled against it")
    return ap.parse_args()


COPY_CALIB_BYTES = 512 << 20


def copy_calibration(torch):
    """torch.neg over a 512 MiB bf16 buffer into another: a streaming kernel
    whose HBM traffic is known exactly (each byte read once, written once)."""
    n = COPY_CALIB_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    return {"kernel": "torch.neg bf16", "bytes_read": COPY_CALIB_BYTES,
            "bytes_written": COPY_CALIB_BYTES}


def visible_pairs(offsets):
    import numpy as np
    L = np.diff(offsets).astype(np.int64)
    return int((L * (L + 1) // 2).sum())


def traffic_record(kernel: str, src: str):
    """HBM bytes per launch from committed counter summaries, valid only while
    the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != h:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, budget_s):
    """The CPU oracle, as it stands, on the first sequences of the same
    workload until ~budget_s of work is done."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    p = w.layers[0]
    tokens = 0
    seqs = 0
    t0 = time.perf_counter()
    for b in range(w.num_seqs):
        s, e = int(w.offsets[b]), int(w.offsets[b + 1])
        oracle.layer(w.x[s:e], p, np.array([0, e - s]), w.timestamps[s:e], w.num_heads,
                     w.n_max, w.alpha, w.ln_eps)
        tokens += e - s
        seqs += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle layer forward on the first {seqs} sequence(s) "
                      f"({tokens} tokens) of the same workload, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(sequences are independent; see the sharding note in the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    hstu.load()
    w = gen.make_config(args.workload)
    dw = runner.DeviceWorkload(w)
    T, d, H = w.total_tokens, w.d_model, w.num_heads
    P = visible_pairs(w.offsets)
    attn_flop = 4.0 * d * P
    lay = dw.layers[0]
    act = dw.act
    mk = lambda dt=act: torch.empty((T, d), dtype=dt, device="cuda")
    u, v, q, k, g, y = mk(), mk(), mk(), mk(), mk(), mk()
    av = mk(torch.float32)
    x = dw.x
    desc, jag = dw.desc, dw.jagged
    attn_ws = hstu.workspace_tensor(hstu.hstu_attn_workspace_size(desc, jag))
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        hstu.hstu_proj_fwd(desc, lay.params, T, x, u, v, q, k, sh)
        rec(1)
        hstu.hstu_attn_fwd(desc, jag, None, q, k, v, lay.pos_bias, lay.time_bias, av, attn_ws, sh)
        rec(2)
        hstu.hstu_norm_gate_fwd(desc, T, av, u, lay.gamma, lay.beta, g, sh)
        rec(3)
        hstu.hstu_out_fwd(desc, T, g, x, lay.w2, lay.b2, y, sh)
        rec(4)

    calib = copy_calibration(torch) if args.copy_calib else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    # per-launch durations (ms) of each kernel, one sample per timed step
    per = {name: np.array([e[j].elapsed_time(e[j + 1]) for e in evs])
           for j, name in enumerate(["proj", "attn", "norm_gate", "out"])}
    steps_ms = np.array([e[0].elapsed_time(e[4]) for e in evs])
    attn_ms = float(np.mean(per["attn"]))
    pct = lambda a: {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
                     "p90": float(np.percentile(a, 90))}

    # cross-check: the same layer through the single hstu_layer_fwd entry point
    ws = dw.workspace()
    y2 = mk()
    for _ in range(2):
        hstu.hstu_layer_fwd(desc, lay.params, jag, None, x, y2, None, None, ws, sh)
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s2.record(stream)
    for _ in range(K):
        hstu.hstu_layer_fwd(desc, lay.params, jag, None, x, y2, None, None, ws, sh)
    e2.record(stream)
    torch.cuda.synchronize()
    layer_ms = s2.elapsed_time(e2) / K
    same = bool(torch.equal(y, y2))

    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    esz = 2
    proj_flop, out_flop = 8.0 * T * d * d, 2.0 * T * d * d
    ng_bytes = T * d * (4 + esz + esz)        # read AV (fp32) and U, write G
    kernels = {
        "proj": {"ms": pct(per["proj"]), "tflops": proj_flop / np.mean(per["proj"]) / 1e9,
                 "pct_bf16_peak": 100 * proj_flop / np.mean(per["proj"]) / 1e9 / PEAK_BF16_TFLOPS},
        "attn": {"ms": pct(per["attn"]), "tflops": attn_tflops,
                 "pct_bf16_peak": 100 * attn_tflops / PEAK_BF16_TFLOPS},
        "norm_gate": {"ms": pct(per["norm_gate"]),
                      "gbs": ng_bytes / np.mean(per["norm_gate"]) / 1e6,
                      "pct_hbm_peak": 100 * ng_bytes / np.mean(per["norm_gate"]) / 1e6 / PEAK_HBM_GBS},
        "out": {"ms": pct(per["out"]), "tflops": out_flop / np.mean(per["out"]) / 1e9,
                "pct_bf16_peak": 100 * out_flop / np.mean(per["out"]) / 1e9 / PEAK_BF16_TFLOPS},
        "step": {"ms": pct(steps_ms)},
    }
    src = os.path.join(ROOT, "hstu_sequential_transducer_jagged_amd", "csrc", "attn.hip")
    rec = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": gen.CONFIG_NAMES[args.workload], "total_tokens": T,
                   "num_seqs": w.num_seqs, "max_seq_len": w.max_seq_len, "d_model": d,
                   "num_heads": H, "head_dim": d // H, "visible_pairs": P},
        "roofline": {"kernel": "attn_bf16", "bound": "mfma", "achieved": attn_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record("attn_bf16", src),
                     "algorithmic_flop_per_launch": attn_flop,
                     "avg_launch_ms": attn_ms},
        "attn_tflops": attn_tflops,
        "attn_pct_bf16_peak": 100.0 * attn_tflops / PEAK_BF16_TFLOPS,
        "hstu_layer_fwd_ms": layer_ms,
        "hstu_layer_fwd_matches_steps": same,
        "kernels": kernels,
    }
    if calib is not None:
        rec["copy_calib"] = calib
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
