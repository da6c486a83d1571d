"""Helpers that compose the C-ABI entry points on the device.

* ``DeviceWorkload``: uploads a workload's arrays (numpy) into device tensors
  (bf16 or fp32 activations and weights, fp32 tables, int64 offsets and
  timestamps). Torch is used for memory and streams only.
* ``layer_forward`` / ``stack_forward``: one layer, or L stacked layers
  (layer l's output is layer l+1's input), optionally starting from the
  action-oriented embedding sum.
* ``ranking_forward``: candidate scoring over a cached history: the history
  runs once through every layer keeping each layer's K and V, then the
  candidates run in micro-batches, all targets, against that cache (M-FALCON
  of "HSTU：Scaling Law 的首次探索" §7.1.5).

Every arithmetic step runs in libhstu.so; this module only allocates and
sequences calls.
"""

from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import hstu


def _torch():
    import torch
    return torch


class DeviceLayer:
    """Device copy of one layer's parameters, with the layer's own descriptor
    (``desc`` with input_norm set when the layer has the input LayerNorm).
    A layer with ``linear_bias`` = (m_p, m_t) gets its position and time
    tables filled on the device by ``hstu_linear_bias_tables``."""

    def __init__(self, p, dtype: int, device, desc=None):
        torch = _torch()
        act = torch.bfloat16 if dtype == hstu.HSTU_BF16 else torch.float32
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        self.w1 = torch.from_numpy(np.ascontiguousarray(p.w1, np.float32)).to(device).to(act)
        self.w2 = torch.from_numpy(np.ascontiguousarray(p.w2, np.float32)).to(device).to(act)
        self.b1 = f32(p.b1)
        self.b2 = f32(p.b2)
        self.gamma = f32(p.gamma)
        self.beta = f32(p.beta)
        self.pos_bias = f32(p.pos_bias)
        self.time_bias = f32(p.time_bias)
        norm1 = bool(getattr(p, "input_norm", False))
        self.ln1_gamma = f32(p.ln1_gamma) if norm1 and getattr(p, "ln1_gamma", None) is not None else None
        self.ln1_beta = f32(p.ln1_beta) if norm1 and getattr(p, "ln1_beta", None) is not None else None
        self.desc = None
        if desc is not None:
            self.desc = hstu.LayerDesc.from_buffer_copy(desc)
            self.desc.input_norm = int(norm1)
            lin = getattr(p, "linear_bias", None)
            if lin is not None:
                hstu.hstu_linear_bias_tables(self.desc, lin[0], lin[1], self.pos_bias, self.time_bias)
        self.params = hstu.make_params(self.w1, self.b1, self.w2, self.b2, self.gamma, self.beta,
                                       self.pos_bias, self.time_bias, self.ln1_gamma, self.ln1_beta)


class DeviceWorkload:
    """Device copy of a workload (see ``hstu_inputs.gen.Workload``)."""

    def __init__(self, w, device="cuda", layers: Optional[List[int]] = None):
        torch = _torch()
        self.w = w
        self.device = device
        self.dtype = hstu.HSTU_BF16 if w.dtype == "bf16" else hstu.HSTU_F32
        self.act = torch.bfloat16 if self.dtype == hstu.HSTU_BF16 else torch.float32
        self.desc = hstu.make_desc(w.d_model, w.num_heads, self.dtype, 2 * w.n_max - 1,
                                   alpha=w.alpha, ln_eps=w.ln_eps,
                                   num_time_buckets=w.num_time_buckets)
        self.offsets = torch.from_numpy(np.asarray(w.offsets, np.int64)).to(device)
        self.timestamps = torch.from_numpy(np.asarray(w.timestamps, np.int64)).to(device)
        self.jagged = hstu.Jagged(w.num_seqs, w.max_seq_len, w.total_tokens,
                                  hstu.ptr(self.offsets), hstu.ptr(self.timestamps), None)
        self.x = None if w.x is None else self.upload_act(w.x)
        idx = range(len(w.layers)) if layers is None else layers
        self.layers = [DeviceLayer(w.layers[i], self.dtype, device, self.desc) for i in idx]
        if w.item_emb is not None:
            self.item_emb = self.upload_act(w.item_emb)
            self.action_emb = self.upload_act(w.action_emb)
            self.item_ids = torch.from_numpy(np.asarray(w.item_ids, np.int64)).to(device)
            self.actions = torch.from_numpy(np.asarray(w.actions, np.int32)).to(device)

    def upload_act(self, a):
        torch = _torch()
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(self.device).to(self.act)

    def empty_act(self, T: int):
        torch = _torch()
        return torch.empty((max(T, 1), self.w.d_model), dtype=self.act, device=self.device)

    def workspace(self, jagged=None):
        """A workspace large enough for every layer (with or without Norm1)."""
        j = jagged or self.jagged
        need = max([hstu.hstu_layer_workspace_size(self.desc, j)] +
                   [hstu.hstu_layer_workspace_size(l.desc, j) for l in self.layers])
        return hstu.workspace_tensor(need, self.device)


def layer_forward(dw: DeviceWorkload, x, layer: int = 0, y=None, workspace=None, jagged=None,
                  cache=None, k_out=None, v_out=None):
    jagged = jagged or dw.jagged
    T = jagged.total_tokens
    y = dw.empty_act(T) if y is None else y
    ws = dw.workspace(jagged) if workspace is None else workspace
    hstu.hstu_layer_fwd(dw.layers[layer].desc, dw.layers[layer].params, jagged, cache, x, y, k_out,
                        v_out, ws)
    return y


def embed_forward(dw: DeviceWorkload, out=None):
    w = dw.w
    x = dw.empty_act(w.total_tokens) if out is None else out
    hstu.hstu_embed_fwd(w.total_tokens, w.d_model, dw.dtype, dw.item_emb, dw.action_emb,
                        dw.item_ids, dw.actions, x)
    return x


def stack_forward(dw: DeviceWorkload, x=None, return_all: bool = False):
    """Embedding (when the workload has tables) then every layer in turn."""
    T = dw.w.total_tokens
    h = embed_forward(dw) if x is None and dw.x is None else (dw.x if x is None else x)
    ws = dw.workspace()
    outs = [h]
    for l in range(len(dw.layers)):
        y = dw.empty_act(T)
        layer_forward(dw, h, l, y=y, workspace=ws)
        outs.append(y)
        h = y
    return outs if return_all else h


def capture(fn, *args, **kwargs):
    """Records fn(*args, **kwargs), a sequence of the library's calls on the
    current stream, into a HIP graph (torch.cuda.CUDAGraph), after one eager
    run on a side stream. Returns (graph, result): graph.replay() re-runs
    every kernel with the same device pointers, so `result` (and any buffer fn
    allocated) holds each replay's output. The calls must not synchronise
    (hstu_check_inputs does); the library's entry points allocate nothing and
    clear memory with kernels, never with memset nodes."""
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(*args, **kwargs)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn(*args, **kwargs)
    return graph, out


class RankingPlan:
    """Candidate rows re-laid out micro-batch-major so that each micro-batch
    is one contiguous jagged batch: [mb0: user0 rows, user1 rows, ...; mb1:
    ...]. ``order`` maps the device row index to the original candidate row."""

    def __init__(self, w, b_m: Optional[int] = None):
        b_m = int(b_m or w.micro_batch)
        cl = np.diff(w.cand_offsets)
        nmb = int(np.max((cl + b_m - 1) // b_m)) if cl.size else 0
        order, mbs = [], []
        start = 0
        for mb in range(nmb):
            lens = []
            for u in range(cl.shape[0]):
                s = int(w.cand_offsets[u]) + mb * b_m
                e = min(int(w.cand_offsets[u + 1]), s + b_m)
                n = max(0, e - s)
                lens.append(n)
                order.extend(range(s, s + n))
            offs = np.zeros(len(lens) + 1, np.int64)
            np.cumsum(lens, out=offs[1:])
            mbs.append((start, offs, int(max(lens) if lens else 0)))
            start += int(offs[-1])
        self.b_m = b_m
        self.order = np.asarray(order, np.int64)
        self.micro_batches = mbs  # (first device row, offsets, max length)


def request_forward(dw: DeviceWorkload, jagged, x, caches=None, workspace=None):
    """One request's own tokens through every layer; layer l also attends to
    ``caches[l]`` (a C cache descriptor) when given. Returns the last layer's
    output and every layer's K and V of these tokens (to cache them)."""
    T = jagged.total_tokens
    L = len(dw.layers)
    ks = [dw.empty_act(T) for _ in range(L)]
    vs = [dw.empty_act(T) for _ in range(L)]
    ws = dw.workspace(jagged) if workspace is None else workspace
    h = x
    for l in range(L):
        y = dw.empty_act(T)
        hstu.hstu_layer_fwd(dw.layers[l].desc, dw.layers[l].params, jagged,
                            None if caches is None else caches[l], h, y, ks[l], vs[l], ws)
        h = y
    return h, ks, vs


class DeviceCache:
    """One layer's K/V cache on the device with its C descriptor (the tensors
    stay referenced while the descriptor is in use)."""

    def __init__(self, offsets, timestamps, k, v, max_len: int, total_tokens: int):
        self.offsets, self.timestamps, self.k, self.v = offsets, timestamps, k, v
        self.c = hstu.KVCache(hstu.ptr(offsets), hstu.ptr(timestamps), hstu.ptr(k), hstu.ptr(v),
                              int(max_len), int(total_tokens))


def concat_caches(dw: DeviceWorkload, a_caches, n_offsets, n_timestamps, n_ks, n_vs,
                  n_total: int, max_len: int):
    """Per layer, the earlier request's cache followed, user by user, by the
    K/V rows of the tokens a later request added (hstu_kv_cache_concat).
    ``max_len`` bounds every user's combined length."""
    torch = _torch()
    B = n_offsets.numel() - 1
    out = []
    for l, a in enumerate(a_caches):
        n = hstu.KVCache(hstu.ptr(n_offsets), hstu.ptr(n_timestamps), hstu.ptr(n_ks[l]),
                         hstu.ptr(n_vs[l]), 0, int(n_total))
        rows = a.c.total_tokens + int(n_total)
        off = torch.empty(B + 1, dtype=torch.int64, device=dw.device)
        ts = torch.empty(max(rows, 1), dtype=torch.int64, device=dw.device)
        k, v = dw.empty_act(rows), dw.empty_act(rows)
        hstu.hstu_kv_cache_concat(dw.layers[l].desc, B, a.c, n, off, ts, k, v)
        out.append(DeviceCache(off, ts, k, v, max_len, rows))
    return out


def score_candidates(dw: DeviceWorkload, plan: RankingPlan, caches, cand_x, cand_ts):
    """Every micro-batch of the plan through all layers against the per-layer
    caches (C descriptors). cand_x / cand_ts: device rows in the plan's
    order. Returns the final outputs in that order."""
    torch = _torch()
    dev = dw.device
    L = len(dw.layers)
    out = torch.empty_like(cand_x)
    keep = []
    for (start, offs, mlen) in plan.micro_batches:
        n = int(offs[-1])
        if n == 0:
            continue
        offs_d = torch.from_numpy(offs).to(dev)
        tgt_d = torch.from_numpy(np.diff(offs).astype(np.int32)).to(dev)
        jag = hstu.Jagged(len(offs) - 1, mlen, n, hstu.ptr(offs_d),
                          hstu.ptr(cand_ts) + 8 * start, hstu.ptr(tgt_d))
        keep.append((offs_d, tgt_d))
        wsc = dw.workspace(jag)
        xin = cand_x[start:start + n]
        for l in range(L):
            y = out[start:start + n] if l == L - 1 else dw.empty_act(n)
            hstu.hstu_layer_fwd(dw.layers[l].desc, dw.layers[l].params, jag, caches[l], xin, y,
                                None, None, wsc)
            xin = y
    torch.cuda.current_stream().synchronize()
    del keep
    return out


def ranking_forward(dw: DeviceWorkload, plan: RankingPlan, keep_history: bool = False):
    """History pass (keeps K, V per layer), then every micro-batch through all
    layers against the cached history. Returns the final candidate outputs in
    the plan's device row order (and the history outputs if asked)."""
    torch = _torch()
    w = dw.w
    dev = dw.device
    Th = w.total_tokens
    L = len(dw.layers)
    kc = [dw.empty_act(Th) for _ in range(L)]
    vc = [dw.empty_act(Th) for _ in range(L)]
    ws = dw.workspace()
    h = dw.x
    hist = [h]
    for l in range(L):
        y = dw.empty_act(Th)
        layer_forward(dw, h, l, y=y, workspace=ws, k_out=kc[l], v_out=vc[l])
        hist.append(y)
        h = y
    cx = dw.upload_act(np.asarray(w.cand_x)[plan.order])
    cts = torch.from_numpy(np.asarray(w.cand_timestamps, np.int64)[plan.order]).to(dev)
    caches = [hstu.make_cache(dw.offsets, dw.timestamps, kc[l], vc[l], w.max_seq_len)
              for l in range(L)]
    out = score_candidates(dw, plan, caches, cx, cts)
    return (out, hist) if keep_history else out
