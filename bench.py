#!/usr/bin/env python3
"""Benchmark: the HSTU layer forward on seeded synthetic jagged workloads.

Default (``--workload 2``, the headline line): 16 sequences with lengths
uniform on [2048, 8192] (the first fixed at 8192), d_model 512, 8 heads of 64,
bf16. A step is one pass of the whole layer path: projection (f1 + SiLU +
split), jagged causal SiLU attention with the position/time bias,
LayerNorm-gate and f2 + residual, each launched through its C-ABI entry point
on one stream, inputs resident in HBM. Steps are timed with HIP events; each
kernel's launches are bracketed by events inside the same timed region.

Other workloads (extra lines; parity is covered by the tests):
  0, 1  one layer as above (fp32 64 tokens; bf16 64 sequences up to 512);
  3     item/action embedding + an 8-layer stack over 128 Zipf-length
        sequences (value = tokens through the whole stack per second);
  4     ranking: 32 users x 4096 history tokens through 4 layers keeping K/V,
        then 512 candidates per user in micro-batches of 128 against that
        cache (value = history + candidate tokens per second).

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
PEAK_F32_TFLOPS = 157.3       # MI355X fp32, matrix cores (dense) and vector alike


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--spin-up-s", type=float, default=0.3,
                    help="untimed seconds of back-to-back steps before the warm-up steps, so "
                         "that the GPU clocks have settled under load when timing starts")
    ap.add_argument("--input-norm", action="store_true",
                    help="layer workloads: apply the input LayerNorm (Norm1) before f1 "
                         "(gamma 1, beta 0, as the default affine recipe)")
    ap.add_argument("--linear-bias", type=str, default=None, metavar="MP,MT",
                    help="layer workloads: parameter-free position/time bias slopes in place "
                         "of the drawn tables (tables filled by hstu_linear_bias_tables)")
    ap.add_argument("--b-m", type=int, default=None,
                    help="ranking workload: candidates per user per micro-batch (default 128)")
    ap.add_argument("--two-requests", type=float, default=None, metavar="F",
                    help="ranking workload: also time a second request per user whose first "
                         "fraction F of the history is already cached (new tokens against the "
                         "cache, hstu_kv_cache_concat, candidates)")
    ap.add_argument("--stochastic-length", type=float, default=None, metavar="ALPHA",
                    help="layer workloads: sample the batch with Stochastic Length (N = n_max) and "
                         "time the layer over the sampled batch against the full one")
    ap.add_argument("--diag-lengths", default=None,
                    help="attention diagnostic: COUNTxLENGTH (e.g. 16x8192, 1x8192), the workload-2 layer "
                         "(bf16, d_model 512, 8 heads, same seeded recipe) on sequences of those lengths")
    ap.add_argument("--backward", action="store_true",
                    help="layer workloads: time the fp32 layer backward pass (hstu_layer_bwd) on the "
                         "workload's shape in fp32")
    ap.add_argument("--attn-bwd-bf16", action="store_true",
                    help="with --backward: the attention backward on the bf16 matrix cores "
                         "(desc.attn_bwd_bf16); the all-fp32 backward is timed beside it")
    ap.add_argument("--gemm-bwd-bf16", action="store_true",
                    help="with --backward: every product of the training layer (f1, and dG, dW2, dW1, dX "
                         "of the backward) on the bf16 matrix cores (desc.gemm_bwd_bf16); the all-fp32 "
                         "backward is timed beside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate CPU seconds for the oracle sample")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured MFMA-loop, copy and clock probes")
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


def measured_peaks():
    """What this GPU reaches beside the published peaks, measured before the
    timed region: a loop of independent bf16 MFMAs with no memory traffic,
    a 1 GiB streaming copy, and the shader clock under the MFMA load
    (libhstu_probe.so)."""
    from hstu_sequential_transducer_jagged_amd import probe
    m = probe.mfma_bf16()
    c = probe.copy_hbm()
    return {"mfma_bf16_tflops": m["tflops"], "mfma_bf16_frac_of_spec": m["tflops"] / PEAK_BF16_TFLOPS,
            "hbm_copy_gbs": c["gbs"], "hbm_copy_frac_of_spec": c["gbs"] / PEAK_HBM_GBS,
            "shader_ghz_under_mfma": m["shader_ghz"],
            "spec": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS, "ghz": 2.4},
            "probes": "MFMA loop: %d workgroups x 4 waves x %d rounds of four independent "
                      "32x32x16 bf16 MFMAs; copy: %d MiB read + written, 16-byte vectors"
                      % (m["groups"], m["iters"], c["bytes"] >> 20)}


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
    threads = oracle_threads()
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


def run_layer(args):
    """Workloads 0-2: one layer. The timed step is one hstu_layer_fwd call
    (the whole layer through its single entry point); a second pass runs the
    same layer through the four per-kernel entry points between HIP events
    for the per-kernel breakdown and the roofline, and must give bitwise the
    same Y."""
    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    if args.diag_lengths:
        cnt, ln = (int(t) for t in args.diag_lengths.lower().split("x"))
        w = gen.make_custom([ln] * cnt, 512, 8, dtype="bf16", seed=1002 + 100_000, n_max=ln,
                            name="bf16 %d x %d (attention diagnostic) d512 h8" % (cnt, ln))
    else:
        w = gen.make_config(args.workload)
    lin = tuple(float(t) for t in args.linear_bias.split(",")) if args.linear_bias else None
    for p in w.layers:
        if args.input_norm:
            p.input_norm = True
            p.ln1_gamma = np.ones(w.d_model, np.float32)
            p.ln1_beta = np.zeros(w.d_model, np.float32)
        if lin is not None:
            p.linear_bias = lin
    dw = runner.DeviceWorkload(w)
    T, d, H = w.total_tokens, w.d_model, w.num_heads
    P = visible_pairs(w.offsets)
    attn_flop = 4.0 * d * P
    lay = dw.layers[0]
    act = dw.act
    mk = lambda dt=act: torch.empty((T, d), dtype=dt, device="cuda")
    u, v, q, k, g, y = mk(), mk(), mk(), mk(), mk(), mk()
    xn = mk() if args.input_norm else None
    av = mk(torch.float32)
    x = dw.x
    desc, jag = lay.desc, dw.jagged
    attn_ws = hstu.workspace_tensor(hstu.hstu_attn_workspace_size(desc, jag))
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    names = (["layernorm"] if args.input_norm else []) + ["proj", "attn", "norm_gate", "out"]

    def step(ev=None):
        i = iter(range(len(names) + 1))
        rec = (lambda: ev[next(i)].record(stream)) if ev is not None else (lambda: None)
        rec()
        xin = x
        if args.input_norm:
            hstu.hstu_layernorm_fwd(desc, T, x, lay.ln1_gamma, lay.ln1_beta, xn, sh)
            rec()
            xin = xn
        hstu.hstu_proj_fwd(desc, lay.params, T, xin, u, v, q, k, sh)
        rec()
        hstu.hstu_attn_fwd(desc, jag, None, q, k, v, lay.pos_bias, lay.time_bias, av, attn_ws, sh)
        rec()
        hstu.hstu_norm_gate_fwd(desc, T, av, u, lay.gamma, lay.beta, g, sh)
        rec()
        hstu.hstu_out_fwd(desc, T, g, x, lay.w2, lay.b2, y, sh)
        rec()

    calib = copy_calibration(torch) if args.copy_calib else None
    peaks = None if args.no_probes else measured_peaks()
    K = args.steps

    # the timed step: the whole layer through hstu_layer_fwd
    ws = dw.workspace()
    y2 = mk()
    ms_step = timed(lambda: hstu.hstu_layer_fwd(desc, lay.params, jag, None, x, y2, None, None, ws, sh),
                    stream, args.warmup, K)
    # the same step replayed from a HIP graph (host launch cost removed)
    graph, y3 = runner.capture(runner.layer_forward, dw, x, 0)
    ms_graph = timed(graph.replay, stream, args.warmup, K)

    # breakdown: the four per-kernel entry points, HIP events between them
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_separate = start.elapsed_time(end) / K
    # per-launch durations (ms) of each kernel, one sample per timed step
    per = {name: np.array([e[j].elapsed_time(e[j + 1]) for e in evs])
           for j, name in enumerate(names)}
    steps_ms = np.array([e[0].elapsed_time(e[len(names)]) for e in evs])
    # the attention launch (hstu_attn_fwd: the scheduling pass and the
    # kernel) in context, without events between launches: K rounds of
    # [f1, attention] less K rounds of f1 alone, so that the attention reads
    # Q, K, V just written by f1 (back to back on the same inputs they would
    # stay in the caches), and the breakdown's events do not add their gaps
    def proj_only():
        hstu.hstu_proj_fwd(desc, lay.params, T, x, u, v, q, k, sh)

    def proj_attn():
        proj_only()
        hstu.hstu_attn_fwd(desc, jag, None, q, k, v, lay.pos_bias, lay.time_bias, av, attn_ws, sh)
    attn_ms = (timed(proj_attn, stream, args.warmup, K) - timed(proj_only, stream, args.warmup, K))
    pct = lambda a: {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
                     "p90": float(np.percentile(a, 90))}

    same = bool(torch.equal(y, y2))

    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    esz = 2 if w.dtype == "bf16" else 4
    # the attention's compulsory HBM traffic: Q, K, V and the timestamps read
    # once, AV (fp32) written once; the bias tables and offsets are noise
    attn_bytes = T * d * 3 * esz + 8 * T + 4 * T * d
    attn_gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
    proj_flop, out_flop = 8.0 * T * d * d, 2.0 * T * d * d
    ng_bytes = T * d * (4 + esz + esz)        # read AV (fp32) and U, write G
    # both paths run on the matrix cores: bf16 MFMA, and fp32 16x16x4 MFMA
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    kernels = {
        "proj": {"ms": pct(per["proj"]), "tflops": proj_flop / np.mean(per["proj"]) / 1e9,
                 "pct_peak": 100 * proj_flop / np.mean(per["proj"]) / 1e9 / peak},
        "attn": {"ms": pct(per["attn"]), "in_context_ms": attn_ms, "tflops": attn_tflops,
                 "pct_peak": 100 * attn_tflops / peak,
                 "algorithmic_bytes": attn_bytes, "gbs": attn_gbs,
                 "pct_hbm_peak": 100 * attn_gbs / PEAK_HBM_GBS},
        "norm_gate": {"ms": pct(per["norm_gate"]),
                      "gbs": ng_bytes / np.mean(per["norm_gate"]) / 1e6,
                      "pct_hbm_peak": 100 * ng_bytes / np.mean(per["norm_gate"]) / 1e6 / PEAK_HBM_GBS},
        "out": {"ms": pct(per["out"]), "tflops": out_flop / np.mean(per["out"]) / 1e9,
                "pct_peak": 100 * out_flop / np.mean(per["out"]) / 1e9 / peak},
        "step": {"ms": pct(steps_ms)},
        **({"layernorm": {"ms": pct(per["layernorm"]),
                          "gbs": 2 * T * d * esz / np.mean(per["layernorm"]) / 1e6,
                          "pct_hbm_peak": 100 * 2 * T * d * esz / np.mean(per["layernorm"]) / 1e6
                                          / PEAK_HBM_GBS}} if args.input_norm else {}),
    }
    src = os.path.join(ROOT, "hstu_sequential_transducer_jagged_amd", "csrc", "attn.hip")
    rec = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "spin_up_s": args.spin_up_s,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": w.name if args.diag_lengths else gen.CONFIG_NAMES[args.workload],
                   "total_tokens": T,
                   "num_seqs": w.num_seqs, "max_seq_len": w.max_seq_len, "d_model": d,
                   "num_heads": H, "head_dim": d // H, "visible_pairs": P,
                   "input_norm": bool(args.input_norm),
                   "bias": ("parameter-free m_p=%g m_t=%g" % lin) if lin else "tables"},
        "roofline": (
            # short sequences (workload 1): each key tile serves few queries, so the
            # attention is bound by its compulsory HBM traffic, not the matrix cores
            {"kernel": "attn_" + w.dtype, "bound": "hbm", "achieved": attn_gbs,
             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": attn_gbs / PEAK_HBM_GBS,
             "traffic": None, "algorithmic_bytes_per_launch": attn_bytes,
             "avg_launch_ms": attn_ms}
            if args.workload == 1 and not args.diag_lengths else
            {"kernel": "attn_" + w.dtype, "bound": "mfma",
             "achieved": attn_tflops, "peak": peak, "unit": "TFLOP/s",
             "frac": attn_tflops / peak,
             "traffic": (traffic_record("attn_bf16", src)
                         if args.workload == 2 and not args.diag_lengths else None),
             "algorithmic_flop_per_launch": attn_flop,
             "avg_launch_ms": attn_ms}),
        "attn_tflops": attn_tflops,
        "attn_pct_peak": 100.0 * attn_tflops / peak,
        "step_entry_point": "hstu_layer_fwd",
        "separate_entry_points_ms_per_step": ms_separate,
        "separate_entry_points_match_bitwise": same,
        "graph_ms_per_step": ms_graph,
        "graph_matches_bitwise": bool(torch.equal(y3, y2)),
        "kernels": kernels,
    }
    if peaks is not None:
        rec["measured_peaks"] = peaks
        if w.dtype == "bf16":
            rec["roofline"]["frac_of_measured_peak"] = (
                attn_gbs / peaks["hbm_copy_gbs"] if rec["roofline"]["bound"] == "hbm"
                else attn_tflops / peaks["mfma_bf16_tflops"])
    if calib is not None:
        rec["copy_calib"] = calib
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    return rec


SPIN_UP_S = 0.3


def spin_up(step, seconds):
    """Untimed calls of step() for about `seconds` of wall time. Under a
    sudden load the GPU needs some tens of milliseconds before its clocks
    settle, and the first calls in a process also load code objects; a few
    warm-up steps of ~1 ms do not cover that."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def timed(step, stream, warmup, steps):
    """Mean ms of `steps` calls of step() between HIP events on `stream`,
    after the spin-up and `warmup` untimed calls."""
    import torch
    spin_up(step, SPIN_UP_S)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(steps):
        step()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def base_record(args, metric, value, unit, ms, dtype, config):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "spin_up_s": args.spin_up_s, "ms_per_step": ms,
            "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded; no dataset)", "config": config}


def run_stack(args):
    """Workload 3: embedding, then the 8-layer stack, through hstu_embed_fwd and
    hstu_layer_fwd (one workspace, two ping-pong activation buffers)."""
    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    w = gen.make_config(3)
    dw = runner.DeviceWorkload(w)
    T, d, L = w.total_tokens, w.d_model, len(w.layers)
    x0 = dw.empty_act(T)
    bufs = [dw.empty_act(T), dw.empty_act(T)]
    ws = dw.workspace()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step():
        hstu.hstu_embed_fwd(T, d, dw.dtype, dw.item_emb, dw.action_emb, dw.item_ids, dw.actions, x0, sh)
        h = x0
        for l in range(L):
            y = bufs[l % 2]
            hstu.hstu_layer_fwd(dw.layers[l].desc, dw.layers[l].params, dw.jagged, None, h, y, None, None, ws, sh)
            h = y

    ms = timed(step, stream, args.warmup, args.steps)
    P = visible_pairs(w.offsets)
    rec = base_record(args, "HSTU stack fwd tokens/s (embedding + 8 layers), 1 GPU", T / (ms * 1e-3),
                      "tokens/s", ms, w.dtype,
                      {"workload": gen.CONFIG_NAMES[3], "total_tokens": T, "num_seqs": w.num_seqs,
                       "max_seq_len": w.max_seq_len, "layers": L, "d_model": d,
                       "num_heads": w.num_heads, "visible_pairs_per_layer": P})
    rec["layer_tokens_per_s"] = T * L / (ms * 1e-3)
    rec["attn_flop_per_layer"] = 4.0 * d * P
    rec["roofline"] = None
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_stack(w, args.cpu_budget_s)
    return rec


def run_backward(args):
    """The layer backward pass (hstu_layer_bwd: forward recompute, then every
    gradient) on a single-layer workload's shape, in fp32 (the backward's
    dtype), against the fp32 forward of the same layer."""
    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    w = gen.make_config(args.workload)
    w.dtype = "f32"                      # bf16-valued inputs, held and computed in fp32
    if args.input_norm:
        for p in w.layers:
            p.input_norm = True
            p.ln1_gamma = np.ones(w.d_model, np.float32)
            p.ln1_beta = np.zeros(w.d_model, np.float32)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    T, d = w.total_tokens, w.d_model
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    rng = np.random.default_rng(np.random.SeedSequence(8000 + args.workload))
    dy = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to("cuda")
    dx = torch.empty_like(dy)
    g = [torch.empty(n, dtype=torch.float32, device="cuda") for n in
         (4 * d * d, 4 * d, d * d, d, d, d, 2 * w.n_max - 1, w.num_time_buckets, d, d)]
    grads = hstu.make_grads(*g)
    ms_f32_bwd = None
    if args.attn_bwd_bf16 or args.gemm_bwd_bf16:
        # the fp32 backward first, for comparison; then the timed one with the flags
        ws32 = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, dw.jagged))
        ms_f32_bwd = timed(lambda: hstu.hstu_layer_bwd(lay.desc, lay.params, dw.jagged, dw.x, dy, dx, grads,
                                                       ws32, sh), stream, args.warmup, args.steps)
        del ws32
        lay.desc.attn_bwd_bf16 = int(bool(args.attn_bwd_bf16))
        lay.desc.gemm_bwd_bf16 = int(bool(args.gemm_bwd_bf16))
    ws = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, dw.jagged))
    ms = timed(lambda: hstu.hstu_layer_bwd(lay.desc, lay.params, dw.jagged, dw.x, dy, dx, grads, ws, sh),
               stream, args.warmup, args.steps)
    # the same step in two calls: forward keeping its activations, then the backward from them
    yt = torch.empty_like(dy)

    def train_step():
        hstu.hstu_layer_fwd_train(lay.desc, lay.params, dw.jagged, dw.x, yt, ws, sh)
        hstu.hstu_layer_bwd_after_fwd(lay.desc, lay.params, dw.jagged, dw.x, dy, dx, grads, ws, sh)
    ms_step = timed(train_step, stream, args.warmup, args.steps)
    wsf = dw.workspace()
    y = dw.empty_act(T)
    ms_fwd = timed(lambda: hstu.hstu_layer_fwd(lay.desc, lay.params, dw.jagged, None, dw.x, y, None, None,
                                               wsf, sh), stream, args.warmup, args.steps)
    P = visible_pairs(w.offsets)
    # algorithmic FLOPs: the forward recompute (f1 8Td^2, attention S and AV 4dP) and the
    # backward (dG, dW2 2Td^2 each; dW1, dX 8Td^2 each; attention dP, dV, dQ, dK 8dP)
    flop = 8.0 * T * d * d + 4.0 * d * P + 20.0 * T * d * d + 8.0 * d * P
    # executed: the dQ and the dK/dV kernels each recompute S and dP (another 6dP)
    flop_exec = flop + 6.0 * d * P
    on16 = [n for n, f in (("attention", args.attn_bwd_bf16),
                           ("products", args.gemm_bwd_bf16)) if f]
    rec = base_record(args, "HSTU layer backward tokens/s (fp32, forward recompute included"
                      + (", " + " and ".join(on16) + " on bf16 matrix cores" if on16 else "") + "), 1 GPU",
                      T / (ms * 1e-3), "tokens/s", ms, "f32",
                      {"workload": gen.CONFIG_NAMES[args.workload] + ", held in fp32", "total_tokens": T,
                       "input_norm": bool(args.input_norm),
                       "num_seqs": w.num_seqs, "d_model": d, "num_heads": w.num_heads,
                       "visible_pairs": P})
    rec["forward_fp32_ms"] = ms_fwd
    if ms_f32_bwd is not None:
        rec["attn_bwd_bf16"] = bool(args.attn_bwd_bf16)
        rec["gemm_bwd_bf16"] = bool(args.gemm_bwd_bf16)
        rec["backward_all_fp32_ms"] = ms_f32_bwd
    rec["train_step_two_calls_ms"] = ms_step
    if args.stochastic_length is not None:
        # Stochastic Length on the training pass: the sampler's kept rows of
        # X, dY and the timestamps, gathered on the device, then the same
        # backward over the sampled batch
        alpha = float(args.stochastic_length)
        B = w.num_seqs
        rng = np.random.default_rng(np.random.SeedSequence(7000 + args.workload))
        u, keys = rng.random(B), rng.random(T)
        off, rows = hstu.hstu_stochastic_length(w.offsets, alpha, w.n_max, u, keys)
        n = int(rows.size)
        rows_d = torch.from_numpy(rows).to("cuda")
        off_d = torch.from_numpy(off).to("cuda")
        xs, dys, dxs = (torch.empty((max(n, 1), d), dtype=torch.float32, device="cuda") for _ in range(3))
        tss = torch.empty(max(n, 1), dtype=torch.int64, device="cuda")
        lens = np.diff(off)
        jag_s = hstu.Jagged(B, int(lens.max()) if B else 0, n, hstu.ptr(off_d), hstu.ptr(tss), None)
        ws_s = hstu.workspace_tensor(hstu.hstu_layer_bwd_workspace_size(lay.desc, jag_s))

        def gather():
            hstu.hstu_gather_rows(n, 4 * d, rows_d, T, dw.x, xs, sh)
            hstu.hstu_gather_rows(n, 4 * d, rows_d, T, dy, dys, sh)
            hstu.hstu_gather_rows(n, 8, rows_d, T, dw.timestamps, tss, sh)

        ms_gather = timed(gather, stream, args.warmup, args.steps)
        ms_sl = timed(lambda: hstu.hstu_layer_bwd(lay.desc, lay.params, jag_s, xs, dys, dxs, grads, ws_s, sh),
                      stream, args.warmup, args.steps)
        Ps = visible_pairs(off)
        rec["stochastic_length"] = {"alpha": alpha, "kept_tokens": n, "sparsity_tokens": 1.0 - n / T,
                                    "sparsity_pairs": 1.0 - Ps / P, "gather_ms": ms_gather,
                                    "sampled_backward_ms": ms_sl,
                                    "speedup_vs_full": ms / (ms_sl + ms_gather)}
    rec["backward_over_forward"] = ms / ms_fwd
    rec["algorithmic_flop"] = flop
    rec["executed_flop"] = flop_exec
    rec["executed_tflops"] = flop_exec / (ms * 1e-3) / 1e12
    # the matrix work runs on the fp32 matrix cores, or with both bf16 flags on
    # the bf16 ones (f1 on hi/lo splits included); with one flag it is mixed
    # and is priced against the bf16 peak, the higher of the two
    peak = PEAK_BF16_TFLOPS if (args.attn_bwd_bf16 or args.gemm_bwd_bf16) else PEAK_F32_TFLOPS
    rec["roofline"] = {"kernel": "layer backward (all kernels)", "bound": "mfma",
                       "achieved": flop / (ms * 1e-3) / 1e12, "peak": peak,
                       "unit": "TFLOP/s", "frac": flop / (ms * 1e-3) / 1e12 / peak,
                       "traffic": None}
    return rec


def run_stochastic_length(args):
    """Stochastic Length on a layer workload: the host sampler
    (hstu_stochastic_length, N = n_max, seeded draws) picks the kept rows,
    hstu_gather_rows builds the sampled batch on the device, and one layer
    runs over it. Timed against the same layer over the full batch."""
    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    w = gen.make_config(args.workload)
    alpha = float(args.stochastic_length)
    dw = runner.DeviceWorkload(w)
    lay = dw.layers[0]
    T, B, d = w.total_tokens, w.num_seqs, w.d_model
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ws = dw.workspace()
    y_full = dw.empty_act(T)
    ms_full = timed(lambda: hstu.hstu_layer_fwd(lay.desc, lay.params, dw.jagged, None, dw.x, y_full,
                                                None, None, ws, sh), stream, args.warmup, args.steps)
    rng = np.random.default_rng(np.random.SeedSequence(7000 + args.workload))
    u, keys = rng.random(B), rng.random(T)
    t0 = time.perf_counter()
    off, rows = hstu.hstu_stochastic_length(w.offsets, alpha, w.n_max, u, keys)
    ms_sampler = (time.perf_counter() - t0) * 1e3
    n = int(rows.size)
    rows_d = torch.from_numpy(rows).to("cuda")
    off_d = torch.from_numpy(off).to("cuda")
    xs = dw.empty_act(n)
    ts = torch.empty(max(n, 1), dtype=torch.int64, device="cuda")
    lens = np.diff(off)
    jag = hstu.Jagged(B, int(lens.max()) if B else 0, n, hstu.ptr(off_d), hstu.ptr(ts), None)
    ws_s = dw.workspace(jag)
    ys = dw.empty_act(n)

    def gather():
        hstu.hstu_gather_rows(n, d * (2 if w.dtype == "bf16" else 4), rows_d, T, dw.x, xs, sh)
        hstu.hstu_gather_rows(n, 8, rows_d, T, dw.timestamps, ts, sh)

    ms_gather = timed(gather, stream, args.warmup, args.steps)
    ms_sl = timed(lambda: hstu.hstu_layer_fwd(lay.desc, lay.params, jag, None, xs, ys, None, None,
                                              ws_s, sh), stream, args.warmup, args.steps)
    P, Ps = visible_pairs(w.offsets), visible_pairs(off)
    ms = ms_gather + ms_sl
    rec = base_record(args, METRIC + " (Stochastic Length)", n / (ms * 1e-3), "tokens/s", ms, w.dtype,
                      {"workload": gen.CONFIG_NAMES[args.workload], "total_tokens": T,
                       "num_seqs": B, "d_model": d, "num_heads": w.num_heads,
                       "stochastic_length_alpha": alpha, "n_max": w.n_max,
                       "kept_tokens": n, "kept_length": int(np.floor(w.n_max ** (alpha / 2)))})
    rec["sparsity_pairs"] = 1.0 - Ps / P
    rec["sparsity_tokens"] = 1.0 - n / T
    rec["full_batch_ms"] = ms_full
    rec["sampled_layer_ms"] = ms_sl
    rec["gather_ms"] = ms_gather
    rec["host_sampler_ms"] = ms_sampler
    rec["speedup_vs_full"] = ms_full / ms
    rec["input_tokens_per_s"] = T / (ms * 1e-3)
    rec["roofline"] = None
    return rec


def two_requests(args, w, dw, stream, candidates, ms_recompute):
    """Request 1 holds the first fraction F of every user's history (run
    once, untimed, its K/V cached per layer). The timed request 2 runs the
    remaining history tokens against that cache, appends their K/V to it
    (hstu_kv_cache_concat) and scores the same candidates against the
    combined cache; the alternative recomputes the whole history."""
    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    f = float(args.two_requests)
    L, B, dev = len(dw.layers), w.num_seqs, dw.device
    hl = np.diff(w.offsets)
    l1 = np.minimum((hl * f).astype(np.int64), hl)
    l2 = hl - l1
    r1 = np.concatenate([np.arange(w.offsets[u], w.offsets[u] + l1[u]) for u in range(B)])
    r2 = np.concatenate([np.arange(w.offsets[u] + l1[u], w.offsets[u + 1]) for u in range(B)])
    o1, o2 = gen.make_jagged(l1), gen.make_jagged(l2)
    dev_i64 = lambda a: torch.from_numpy(np.asarray(a, np.int64)).to(dev)
    off1, off2 = dev_i64(o1), dev_i64(o2)
    ts1, ts2 = dev_i64(np.asarray(w.timestamps)[r1]), dev_i64(np.asarray(w.timestamps)[r2])
    x1, x2 = dw.upload_act(np.asarray(w.x)[r1]), dw.upload_act(np.asarray(w.x)[r2])
    T1, T2 = int(o1[-1]), int(o2[-1])
    jag1 = hstu.Jagged(B, int(l1.max()), T1, hstu.ptr(off1), hstu.ptr(ts1), None)
    jag2 = hstu.Jagged(B, int(l2.max()), T2, hstu.ptr(off2), hstu.ptr(ts2), None)
    _, k1, v1 = runner.request_forward(dw, jag1, x1)
    c1 = [runner.DeviceCache(off1, ts1, k1[l], v1[l], int(l1.max()), T1) for l in range(L)]
    k2 = [dw.empty_act(T2) for _ in range(L)]
    v2 = [dw.empty_act(T2) for _ in range(L)]
    n2 = [hstu.KVCache(hstu.ptr(off2), hstu.ptr(ts2), hstu.ptr(k2[l]), hstu.ptr(v2[l]), 0, T2)
          for l in range(L)]
    rows = T1 + T2
    c12 = [runner.DeviceCache(torch.empty(B + 1, dtype=torch.int64, device=dev),
                              torch.empty(rows, dtype=torch.int64, device=dev),
                              dw.empty_act(rows), dw.empty_act(rows), int(hl.max()), rows)
           for _ in range(L)]
    ybuf = [dw.empty_act(T2), dw.empty_act(T2)]
    ws2 = dw.workspace(jag2)
    sh = stream.cuda_stream

    def request2():
        h = x2
        for l in range(L):
            hstu.hstu_layer_fwd(dw.layers[l].desc, dw.layers[l].params, jag2, c1[l].c, h, ybuf[l % 2],
                                k2[l], v2[l], ws2, sh)
            h = ybuf[l % 2]
        for l in range(L):
            c = c12[l]
            hstu.hstu_kv_cache_concat(dw.layers[l].desc, B, c1[l].c, n2[l], c.offsets, c.timestamps,
                                      c.k, c.v, sh)
        candidates([c.c for c in c12])

    ms_reuse = timed(request2, stream, args.warmup, args.steps)
    return {"cached_fraction": f, "new_history_tokens": T2, "cached_history_tokens": T1,
            "request2_reuse_ms": ms_reuse, "request2_recompute_ms": ms_recompute,
            "speedup": ms_recompute / ms_reuse}


def cpu_baseline_stack(w, budget_s):
    """The CPU oracle (embedding + every layer) on the first sequences of the
    same workload until ~budget_s of work is done."""
    import numpy as np

    import oracle
    threads = oracle_threads()
    tokens = seqs = 0
    t0 = time.perf_counter()
    for b in range(w.num_seqs):
        s, e = int(w.offsets[b]), int(w.offsets[b + 1])
        x = oracle.embed(w.item_emb, w.action_emb, w.item_ids[s:e], w.actions[s:e])
        oracle.stack(x, w.layers, np.array([0, e - s]), w.timestamps[s:e], w.num_heads, w.n_max,
                     w.alpha, w.ln_eps)
        tokens += e - s
        seqs += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 NumPy oracle: embedding + {len(w.layers)} layers on the first "
                      f"{seqs} sequence(s) ({tokens} tokens) of the same workload, {dt:.1f} s"}


def run_ranking(args):
    """Workload 4: history pass through every layer keeping K/V, then every
    candidate micro-batch through every layer against that cache (all
    device-resident; the micro-batch plan is built once, outside the timing)."""
    import numpy as np
    import torch

    from hstu_inputs import gen
    from hstu_sequential_transducer_jagged_amd import hstu, runner

    w = gen.make_config(4)
    dw = runner.DeviceWorkload(w)
    Th, d, L = w.total_tokens, w.d_model, len(w.layers)
    plan = runner.RankingPlan(w, args.b_m)
    dev = dw.device
    kc = [dw.empty_act(Th) for _ in range(L)]
    vc = [dw.empty_act(Th) for _ in range(L)]
    hbuf = [dw.empty_act(Th), dw.empty_act(Th)]
    ws = dw.workspace()
    cx = dw.upload_act(np.asarray(w.cand_x)[plan.order])
    cts = torch.from_numpy(np.asarray(w.cand_timestamps, np.int64)[plan.order]).to(dev)
    caches = [hstu.make_cache(dw.offsets, dw.timestamps, kc[l], vc[l], w.max_seq_len)
              for l in range(L)]
    mbs = []
    for (start, offs, mlen) in plan.micro_batches:
        n = int(offs[-1])
        if n == 0:
            continue
        offs_d = torch.from_numpy(offs).to(dev)
        tgt_d = torch.from_numpy(np.diff(offs).astype(np.int32)).to(dev)
        jag = hstu.Jagged(len(offs) - 1, mlen, n, hstu.ptr(offs_d), hstu.ptr(cts) + 8 * start,
                          hstu.ptr(tgt_d))
        mbs.append((start, n, jag, offs_d, tgt_d, hstu.workspace_tensor(
            hstu.hstu_layer_workspace_size(dw.desc, jag))))
    Tc = sum(m[1] for m in mbs)
    cbuf = [torch.empty_like(cx), torch.empty_like(cx)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def history():
        h = dw.x
        for l in range(L):
            y = hbuf[l % 2]
            hstu.hstu_layer_fwd(dw.layers[l].desc, dw.layers[l].params, dw.jagged, None, h, y, kc[l], vc[l], ws, sh)
            h = y

    def candidates(cs=caches):
        for (start, n, jag, _, _, wsc) in mbs:
            h = cx[start:start + n]
            for l in range(L):
                y = cbuf[l % 2][start:start + n]
                hstu.hstu_layer_fwd(dw.layers[l].desc, dw.layers[l].params, jag, cs[l], h, y, None, None,
                                    wsc, sh)
                h = y

    def step():
        history()
        candidates()

    ms = timed(step, stream, args.warmup, args.steps)
    ms_h = timed(history, stream, 1, args.steps)
    ms_c = timed(candidates, stream, 1, args.steps)
    rec = base_record(args, "HSTU ranking fwd tokens/s (history + candidates, 4 layers), 1 GPU",
                      (Th + Tc) / (ms * 1e-3), "tokens/s", ms, w.dtype,
                      {"workload": gen.CONFIG_NAMES[4], "history_tokens": Th, "candidates": Tc,
                       "users": w.num_seqs, "layers": L, "micro_batch": plan.b_m,
                       "micro_batches": len(mbs), "d_model": d, "num_heads": w.num_heads})
    rec["history_tokens_per_s"] = Th / (ms_h * 1e-3)
    rec["history_ms"] = ms_h
    rec["candidates_per_s"] = Tc / (ms_c * 1e-3)
    rec["candidates_ms"] = ms_c
    rec["ms_per_micro_batch"] = ms_c / max(len(mbs), 1)   # all layers, all users
    if args.two_requests is not None:
        rec["two_requests"] = two_requests(args, w, dw, stream, candidates, ms)
    rec["roofline"] = None
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_ranking(w, args.cpu_budget_s)
    return rec


def cpu_baseline_ranking(w, budget_s):
    """The CPU oracle's ranking (history through every layer, then every
    candidate micro-batch against the cached history) on the first users of
    the same workload until ~budget_s of work is done."""
    import dataclasses

    import numpy as np

    import oracle
    threads = oracle_threads()
    tokens = users = 0
    t0 = time.perf_counter()
    for u in range(w.num_seqs):
        s, e = int(w.offsets[u]), int(w.offsets[u + 1])
        cs, ce = int(w.cand_offsets[u]), int(w.cand_offsets[u + 1])
        sub = dataclasses.replace(
            w, offsets=np.array([0, e - s], np.int64), timestamps=w.timestamps[s:e], x=w.x[s:e],
            cand_offsets=np.array([0, ce - cs], np.int64),
            cand_timestamps=w.cand_timestamps[cs:ce], cand_x=w.cand_x[cs:ce])
        oracle.ranking(sub)
        tokens += (e - s) + (ce - cs)
        users += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 NumPy oracle ranking (history + candidates, {len(w.layers)} layers) "
                      f"for the first {users} user(s) ({tokens} tokens) of the same workload, "
                      f"{dt:.1f} s"}


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count()


def main():
    args = parse()
    global SPIN_UP_S
    SPIN_UP_S = args.spin_up_s
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path (the sequences of a "
              "batch are independent, so a data-parallel split of the forward needs no "
              "communication between GPUs).", file=sys.stderr)
        sys.exit(2)
    import torch  # noqa: F401  (torch's HIP runtime first, then the library bound to it)

    from hstu_sequential_transducer_jagged_amd import hstu
    hstu.load()
    if (args.input_norm or args.linear_bias) and args.workload in (3, 4):
        print("--input-norm and --linear-bias apply to the single-layer workloads 0-2",
              file=sys.stderr)
        sys.exit(2)
    if args.stochastic_length is not None and args.workload in (3, 4):
        print("--stochastic-length applies to the single-layer workloads 0-2", file=sys.stderr)
        sys.exit(2)
    run = {3: run_stack, 4: run_ranking}.get(args.workload, run_layer)
    if args.stochastic_length is not None:
        run = run_stochastic_length
    if args.backward:
        if args.workload in (3, 4):
            print("--backward applies to the single-layer workloads 0-2", file=sys.stderr)
            sys.exit(2)
        run = run_backward
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
