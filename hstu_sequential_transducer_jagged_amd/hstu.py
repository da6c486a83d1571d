"""Thin Python binding of the HIP library ``libhstu.so`` (ctypes).

Argument marshalling only: every step of the layer runs in the library's
gfx950 kernels. Torch tensors serve as device memory and the current torch
stream as the HIP stream. The entry points carry the C names declared in
``include/hstu.h``; a non-zero status raises ``HstuError`` with the
library's message. There is no fallback: if the library is missing, loading
fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu.so")

HSTU_OK = 0
HSTU_E_INVAL = -1
HSTU_E_UNSUPPORTED = -2
HSTU_E_WORKSPACE = -3
HSTU_E_DEVICE = -4
HSTU_E_DATA = -5
HSTU_F32 = 0
HSTU_BF16 = 1
HSTU_BIAS_TABLES = 0
HSTU_BIAS_LINEAR = 1
HSTU_MAX_TOKEN_TYPES = 4

EXPORTS = ("hstu_abi_version", "hstu_last_error", "hstu_proj_fwd", "hstu_attn_workspace_size",
           "hstu_attn_fwd", "hstu_attn_fwd_noalloc",
           "hstu_norm_gate_fwd", "hstu_layernorm_fwd", "hstu_linear_bias_tables",
           "hstu_kv_cache_concat", "hstu_stochastic_length", "hstu_gather_rows",
           "hstu_out_fwd", "hstu_layer_workspace_size",
           "hstu_layer_fwd", "hstu_layer_bwd_workspace_size", "hstu_layer_bwd",
           "hstu_layer_fwd_train", "hstu_layer_bwd_after_fwd",
           "hstu_embed_fwd", "hstu_check_inputs")


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hstu status {status}: {message}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("ln_eps", ctypes.c_float),
                ("pos_table_len", ctypes.c_int32), ("num_time_buckets", ctypes.c_int32),
                ("input_norm", ctypes.c_int32), ("target_no_self", ctypes.c_int32),
                ("num_token_types", ctypes.c_int32), ("bias_mode", ctypes.c_int32),
                ("linear_m_p", ctypes.c_float), ("linear_m_t", ctypes.c_float),
                ("attn_bwd_bf16", ctypes.c_int32), ("gemm_bwd_bf16", ctypes.c_int32)]


class Jagged(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("offsets", ctypes.c_void_p),
                ("timestamps", ctypes.c_void_p), ("num_targets", ctypes.c_void_p),
                ("token_types", ctypes.c_void_p)]


class KVCache(ctypes.Structure):
    _fields_ = [("offsets", ctypes.c_void_p), ("timestamps", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("max_len", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("token_types", ctypes.c_void_p)]


class LayerParams(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("ln_gamma", ctypes.c_void_p),
                ("ln_beta", ctypes.c_void_p), ("pos_bias", ctypes.c_void_p),
                ("time_bias", ctypes.c_void_p), ("ln1_gamma", ctypes.c_void_p),
                ("ln1_beta", ctypes.c_void_p)]


class LayerGrads(ctypes.Structure):
    _fields_ = [("dw1", ctypes.c_void_p), ("db1", ctypes.c_void_p), ("dw2", ctypes.c_void_p),
                ("db2", ctypes.c_void_p), ("dgamma", ctypes.c_void_p), ("dbeta", ctypes.c_void_p),
                ("dpos", ctypes.c_void_p), ("dtime", ctypes.c_void_p),
                ("dln1_gamma", ctypes.c_void_p), ("dln1_beta", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhstu.so (built in-tree by ``build()``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build the HIP library first "
                           "(python -m hstu_sequential_transducer_jagged_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    sig = {
        "hstu_abi_version": (ctypes.c_int, []),
        "hstu_last_error": (ctypes.c_char_p, []),
        "hstu_proj_fwd": (ctypes.c_int, [P, P, i64, P, P, P, P, P, P]),
        "hstu_attn_workspace_size": (ctypes.c_size_t, [P, P]),
        "hstu_attn_fwd": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "hstu_attn_fwd_noalloc": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P]),
        "hstu_norm_gate_fwd": (ctypes.c_int, [P, i64, P, P, P, P, P, P]),
        "hstu_layernorm_fwd": (ctypes.c_int, [P, i64, P, P, P, P, P]),
        "hstu_linear_bias_tables": (ctypes.c_int, [P, ctypes.c_float, ctypes.c_float, P, P, P]),
        "hstu_kv_cache_concat": (ctypes.c_int, [P, i32, P, P, P, P, P, P, P]),
        "hstu_stochastic_length": (ctypes.c_int, [i32, P, ctypes.c_double, i64, P, P, P, P, i64, P]),
        "hstu_gather_rows": (ctypes.c_int, [i64, i32, P, i64, P, P, P]),
        "hstu_out_fwd": (ctypes.c_int, [P, i64, P, P, P, P, P, P]),
        "hstu_layer_workspace_size": (ctypes.c_size_t, [P, P]),
        "hstu_layer_fwd": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "hstu_layer_bwd_workspace_size": (ctypes.c_size_t, [P, P]),
        "hstu_layer_bwd": (ctypes.c_int, [P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "hstu_layer_fwd_train": (ctypes.c_int, [P, P, P, P, P, P, ctypes.c_size_t, P]),
        "hstu_layer_bwd_after_fwd": (ctypes.c_int, [P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "hstu_embed_fwd": (ctypes.c_int, [i64, i32, i32, P, i64, P, i32, P, P, P, P]),
        "hstu_check_inputs": (ctypes.c_int, [P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != HSTU_OK:
        raise HstuError(status, load().hstu_last_error().decode())


def _ref(s):
    return None if s is None else ctypes.byref(s)


def ptr(t) -> Optional[int]:
    """Device address of a tensor (or None)."""
    return None if t is None else t.data_ptr()


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# descriptors built from tensors (marshalling only)
# ---------------------------------------------------------------------------

def make_desc(d_model: int, num_heads: int, dtype: int, pos_table_len: int,
              alpha: float = 1.0, ln_eps: float = 1e-5, num_time_buckets: int = 32,
              input_norm: bool = False, target_no_self: bool = False,
              num_token_types: int = 0, bias_mode: int = HSTU_BIAS_TABLES,
              linear_m_p: float = 0.0, linear_m_t: float = 0.0,
              attn_bwd_bf16: bool = False, gemm_bwd_bf16: bool = False) -> LayerDesc:
    return LayerDesc(d_model, num_heads, d_model // num_heads, dtype, alpha, ln_eps,
                     pos_table_len, num_time_buckets, int(bool(input_norm)), int(bool(target_no_self)),
                     int(num_token_types), int(bias_mode), float(linear_m_p), float(linear_m_t),
                     int(bool(attn_bwd_bf16)), int(bool(gemm_bwd_bf16)))


def make_jagged(offsets, timestamps, max_seq_len: int, num_targets=None,
                token_types=None) -> Jagged:
    """offsets: int64 device tensor [B+1]; timestamps: int64 device [T];
    num_targets: int32 device [B] or None; token_types: int32 device [T] or None."""
    B = offsets.numel() - 1
    T = int(offsets[-1].item()) if B > 0 else 0
    return Jagged(B, int(max_seq_len), T, ptr(offsets), ptr(timestamps), ptr(num_targets),
                  ptr(token_types))


def make_cache(offsets, timestamps, k, v, max_len: int, token_types=None) -> KVCache:
    T = int(offsets[-1].item()) if offsets.numel() > 1 else 0
    return KVCache(ptr(offsets), ptr(timestamps), ptr(k), ptr(v), int(max_len), T,
                   ptr(token_types))


def make_params(w1, b1, w2, b2, gamma, beta, pos_bias, time_bias, ln1_gamma=None,
                ln1_beta=None) -> LayerParams:
    return LayerParams(ptr(w1), ptr(b1), ptr(w2), ptr(b2), ptr(gamma), ptr(beta),
                       ptr(pos_bias), ptr(time_bias), ptr(ln1_gamma), ptr(ln1_beta))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def hstu_abi_version() -> int:
    return load().hstu_abi_version()


def hstu_proj_fwd(desc, params, T, x, u, v, q, k, stream=None) -> None:
    _check(load().hstu_proj_fwd(_ref(desc), _ref(params), int(T), ptr(x), ptr(u), ptr(v),
                                ptr(q), ptr(k), stream if stream is not None else current_stream()))


def hstu_attn_workspace_size(desc, jagged) -> int:
    return int(load().hstu_attn_workspace_size(_ref(desc), _ref(jagged)))


def hstu_attn_fwd(desc, jagged, cache, q, k, v, pos_bias, time_bias, av, workspace,
                  stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().hstu_attn_fwd(_ref(desc), _ref(jagged), _ref(cache), ptr(q), ptr(k), ptr(v),
                                ptr(pos_bias), ptr(time_bias), ptr(av), ptr(workspace), nbytes,
                                stream if stream is not None else current_stream()))


def hstu_attn_fwd_noalloc(desc, jagged, cache, q, k, v, pos_bias, time_bias, av, stream=None) -> None:
    _check(load().hstu_attn_fwd_noalloc(_ref(desc), _ref(jagged), _ref(cache), ptr(q), ptr(k), ptr(v),
                                        ptr(pos_bias), ptr(time_bias), ptr(av),
                                        stream if stream is not None else current_stream()))


def hstu_norm_gate_fwd(desc, T, av, u, gamma, beta, g, stream=None) -> None:
    _check(load().hstu_norm_gate_fwd(_ref(desc), int(T), ptr(av), ptr(u), ptr(gamma), ptr(beta),
                                     ptr(g), stream if stream is not None else current_stream()))


def hstu_layernorm_fwd(desc, T, x, gamma, beta, y, stream=None) -> None:
    _check(load().hstu_layernorm_fwd(_ref(desc), int(T), ptr(x), ptr(gamma), ptr(beta), ptr(y),
                                     stream if stream is not None else current_stream()))


def hstu_linear_bias_tables(desc, m_p, m_t, pos_bias, time_bias, stream=None) -> None:
    _check(load().hstu_linear_bias_tables(_ref(desc), float(m_p), float(m_t), ptr(pos_bias),
                                          ptr(time_bias),
                                          stream if stream is not None else current_stream()))


def hstu_kv_cache_concat(desc, num_seqs, a, n, out_offsets, out_timestamps, out_k, out_v,
                         stream=None) -> None:
    _check(load().hstu_kv_cache_concat(_ref(desc), int(num_seqs), _ref(a), _ref(n), ptr(out_offsets),
                                       ptr(out_timestamps), ptr(out_k), ptr(out_v),
                                       stream if stream is not None else current_stream()))


def hstu_stochastic_length(offsets, alpha, n_max, u, keys):
    """Host arrays in, (out_offsets, rows) numpy int64 arrays out."""
    import numpy as np
    off = np.ascontiguousarray(offsets, np.int64)
    B = off.shape[0] - 1
    T = int(off[-1]) if B >= 0 else 0
    uu = np.ascontiguousarray(u, np.float64)
    kk = np.ascontiguousarray(keys, np.float64)
    out_off = np.zeros(B + 1, np.int64)
    rows = np.zeros(max(T, 1), np.int64)
    total = ctypes.c_int64(0)
    addr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(load().hstu_stochastic_length(B, addr(off), float(alpha), int(n_max), addr(uu), addr(kk),
                                         addr(out_off), addr(rows), T, ctypes.byref(total)))
    return out_off, rows[:total.value].copy()


def hstu_gather_rows(n, row_bytes, rows, src_rows, src, dst, stream=None) -> None:
    _check(load().hstu_gather_rows(int(n), int(row_bytes), ptr(rows), int(src_rows), ptr(src), ptr(dst),
                                   stream if stream is not None else current_stream()))


def hstu_out_fwd(desc, T, g, x, w2, b2, y, stream=None) -> None:
    _check(load().hstu_out_fwd(_ref(desc), int(T), ptr(g), ptr(x), ptr(w2), ptr(b2), ptr(y),
                               stream if stream is not None else current_stream()))


def hstu_layer_workspace_size(desc, jagged) -> int:
    return int(load().hstu_layer_workspace_size(_ref(desc), _ref(jagged)))


def workspace_tensor(nbytes: int, device="cuda"):
    """Device buffer for a workspace (torch allocations are 256-byte aligned)."""
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def hstu_layer_fwd(desc, params, jagged, cache, x, y, k_out, v_out, workspace,
                   stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().hstu_layer_fwd(_ref(desc), _ref(params), _ref(jagged), _ref(cache), ptr(x),
                                 ptr(y), ptr(k_out), ptr(v_out), ptr(workspace), nbytes,
                                 stream if stream is not None else current_stream()))


def make_grads(dw1, db1, dw2, db2, dgamma, dbeta, dpos, dtime, dln1_gamma=None,
               dln1_beta=None) -> LayerGrads:
    return LayerGrads(ptr(dw1), ptr(db1), ptr(dw2), ptr(db2), ptr(dgamma), ptr(dbeta), ptr(dpos),
                      ptr(dtime), ptr(dln1_gamma), ptr(dln1_beta))


def hstu_layer_bwd_workspace_size(desc, jagged) -> int:
    return load().hstu_layer_bwd_workspace_size(_ref(desc), _ref(jagged))


def hstu_layer_bwd(desc, params, jagged, x, dy, dx, grads, workspace, stream=None) -> None:
    _check(load().hstu_layer_bwd(_ref(desc), _ref(params), _ref(jagged), ptr(x), ptr(dy), ptr(dx),
                                 _ref(grads), ptr(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 stream if stream is not None else current_stream()))


def hstu_layer_fwd_train(desc, params, jagged, x, y, workspace, stream=None) -> None:
    _check(load().hstu_layer_fwd_train(_ref(desc), _ref(params), _ref(jagged), ptr(x), ptr(y),
                                       ptr(workspace),
                                       0 if workspace is None else workspace.numel() * workspace.element_size(),
                                       stream if stream is not None else current_stream()))


def hstu_layer_bwd_after_fwd(desc, params, jagged, x, dy, dx, grads, workspace, stream=None) -> None:
    _check(load().hstu_layer_bwd_after_fwd(_ref(desc), _ref(params), _ref(jagged), ptr(x), ptr(dy),
                                           ptr(dx), _ref(grads), ptr(workspace),
                                           0 if workspace is None else workspace.numel() * workspace.element_size(),
                                           stream if stream is not None else current_stream()))


def hstu_embed_fwd(T, d_model, dtype, item_emb, action_emb, item_ids, actions, x,
                   stream=None) -> None:
    _check(load().hstu_embed_fwd(int(T), int(d_model), int(dtype), ptr(item_emb),
                                 int(item_emb.shape[0]), ptr(action_emb),
                                 int(action_emb.shape[0]), ptr(item_ids), ptr(actions), ptr(x),
                                 stream if stream is not None else current_stream()))


def hstu_check_inputs(desc, jagged, cache=None, stream=None) -> None:
    _check(load().hstu_check_inputs(_ref(desc), _ref(jagged), _ref(cache),
                                    stream if stream is not None else current_stream()))
