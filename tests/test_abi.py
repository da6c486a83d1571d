"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point the header declares, and rejects bad arguments before touching
the device."""

import ctypes
import os
import re

import pytest

from hstu_sequential_transducer_jagged_amd import hstu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hstu.LIB_PATH):
        from hstu_sequential_transducer_jagged_amd import build
        build.build()
    return hstu.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(hstu_\w+)\s*\(", text,
                                 re.MULTILINE)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(hstu.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.hstu_abi_version() == 11


def _desc(**kw):
    d = dict(d_model=512, num_heads=8, dtype=hstu.HSTU_BF16, pos_table_len=255)
    d.update(kw)
    return hstu.make_desc(d["d_model"], d["num_heads"], d["dtype"], d["pos_table_len"])


FAKE = 0x100000   # never dereferenced: validation rejects or returns before any launch


def _attn(lib, desc, jag, cache=None, ptrs=FAKE):
    P = ctypes.c_void_p
    return lib.hstu_attn_fwd(ctypes.byref(desc) if desc else None,
                             ctypes.byref(jag) if jag else None,
                             ctypes.byref(cache) if cache else None,
                             P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(ptrs),
                             P(FAKE), 1 << 20, None)


def _jag(B=2, T=10, mx=6):
    return hstu.Jagged(B, mx, T, FAKE, FAKE, None)


def test_validation_errors(lib):
    assert _attn(lib, None, _jag()) == hstu.HSTU_E_INVAL
    assert b"desc" in lib.hstu_last_error()
    d = _desc()
    d.head_dim = 32
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL          # d_model != H * dh
    d = hstu.make_desc(256, 16, hstu.HSTU_BF16, 255)           # dh = 16
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_UNSUPPORTED
    d = _desc()
    d.dtype = 7
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    for alpha in (0.0, float("nan"), 1e9):
        d = _desc()
        d.alpha = alpha
        assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc()
    d.pos_table_len = 256                                       # even
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc()
    d.num_time_buckets = 0
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc(pos_table_len=9)                                  # n_max 5 < max_seq_len 6
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    assert b"position table" in lib.hstu_last_error()
    cache = hstu.KVCache(FAKE, FAKE, FAKE, FAKE, 125, 100)     # 6 + 125 > 128
    assert _attn(lib, _desc(), _jag(), cache) == hstu.HSTU_E_INVAL
    assert _attn(lib, _desc(), _jag(B=-1)) == hstu.HSTU_E_INVAL
    assert _attn(lib, _desc(), _jag(), ptrs=FAKE + 8) == hstu.HSTU_E_INVAL   # misaligned
    assert _attn(lib, _desc(), _jag(), ptrs=0) == hstu.HSTU_E_INVAL          # NULL


def test_empty_batches_return_ok_without_device(lib):
    assert _attn(lib, _desc(), _jag(B=0, T=0, mx=0)) == hstu.HSTU_OK
    assert _attn(lib, _desc(), _jag(B=3, T=0, mx=0)) == hstu.HSTU_OK
    P = ctypes.c_void_p
    params = hstu.LayerParams(FAKE, None, FAKE, None, None, None, FAKE, FAKE)
    assert lib.hstu_proj_fwd(ctypes.byref(_desc()), ctypes.byref(params), 0, None, None, None,
                             None, None, None) == hstu.HSTU_OK
    assert lib.hstu_proj_fwd(ctypes.byref(_desc()), ctypes.byref(params), -1, None, None, None,
                             None, None, None) == hstu.HSTU_E_INVAL
    assert lib.hstu_norm_gate_fwd(ctypes.byref(_desc()), 0, None, None, None, None, None,
                                  None) == hstu.HSTU_OK
    assert lib.hstu_out_fwd(ctypes.byref(_desc()), 5, P(FAKE), P(FAKE), P(FAKE), None,
                            P(FAKE), None) == hstu.HSTU_E_INVAL   # y aliases x
    assert lib.hstu_embed_fwd(0, 512, hstu.HSTU_BF16, None, 0, None, 0, None, None, None,
                              None) == hstu.HSTU_OK
    assert lib.hstu_embed_fwd(4, 12, hstu.HSTU_BF16, P(FAKE), 1, P(FAKE), 1, P(FAKE), P(FAKE),
                              P(FAKE), None) == hstu.HSTU_E_UNSUPPORTED


def test_layer_workspace_checks(lib):
    d = _desc()
    need = lib.hstu_layer_workspace_size(ctypes.byref(d), ctypes.byref(_jag()))
    attn = lib.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(_jag()))
    # 2 items (< 512) -> 8 key-range splits: work list 4 * (9 + 2 * 8) bytes
    # rounded to 256, then 8 partial outputs of T x d fp32
    assert attn == 256 + 8 * 10 * 512 * 4
    assert need == 4 * 10240 + 20480 + attn
    f = hstu.make_desc(64, 2, hstu.HSTU_F32, 255)
    assert lib.hstu_attn_workspace_size(ctypes.byref(f), ctypes.byref(_jag())) == 0
    P = ctypes.c_void_p
    st = lib.hstu_attn_fwd(ctypes.byref(d), ctypes.byref(_jag()), None, P(FAKE), P(FAKE), P(FAKE),
                           P(FAKE), P(FAKE), P(FAKE), P(FAKE), attn - 1, None)
    assert st == hstu.HSTU_E_WORKSPACE
    params = hstu.LayerParams(FAKE, None, FAKE, None, None, None, FAKE, FAKE)
    P = ctypes.c_void_p
    st = lib.hstu_layer_fwd(ctypes.byref(d), ctypes.byref(params), ctypes.byref(_jag()), None,
                            P(FAKE), P(FAKE + 4096), None, None, P(FAKE), need - 1, None)
    assert st == hstu.HSTU_E_WORKSPACE
    st = lib.hstu_layer_fwd(ctypes.byref(d), ctypes.byref(params), ctypes.byref(_jag()), None,
                            P(FAKE), P(FAKE + 4096), None, None, P(FAKE + 16), need, None)
    assert st == hstu.HSTU_E_INVAL                             # workspace not 256-aligned
    st = lib.hstu_layer_fwd(ctypes.byref(d), ctypes.byref(params), ctypes.byref(_jag()), None,
                            P(FAKE), P(FAKE), None, None, P(FAKE), need, None)
    assert st == hstu.HSTU_E_INVAL                             # y aliases x


def test_option_entry_points_validate(lib):
    """The input LayerNorm and the parameter-free bias tables reject bad
    arguments on the host; an input_norm flag other than 0/1 is refused by
    every entry point, and the layer workspace grows by one [T, d] buffer."""
    P = ctypes.c_void_p
    d = _desc()
    assert lib.hstu_layernorm_fwd(ctypes.byref(d), 0, None, None, None, None, None) == hstu.HSTU_OK
    assert lib.hstu_layernorm_fwd(ctypes.byref(d), 4, P(FAKE), None, None, P(FAKE),
                                  None) == hstu.HSTU_E_INVAL        # y aliases x
    assert lib.hstu_layernorm_fwd(ctypes.byref(d), 4, P(FAKE), P(FAKE + 4), None, P(FAKE + 4096),
                                  None) == hstu.HSTU_E_INVAL        # gamma misaligned
    assert lib.hstu_layernorm_fwd(ctypes.byref(d), -1, P(FAKE), None, None, P(FAKE + 4096),
                                  None) == hstu.HSTU_E_INVAL
    for mp, mt in ((float("nan"), 0.1), (0.1, float("inf"))):
        assert lib.hstu_linear_bias_tables(ctypes.byref(d), mp, mt, P(FAKE), P(FAKE + 4096),
                                           None) == hstu.HSTU_E_INVAL
    assert lib.hstu_linear_bias_tables(ctypes.byref(d), 0.1, 0.1, P(FAKE), P(FAKE),
                                       None) == hstu.HSTU_E_INVAL   # tables alias
    assert lib.hstu_linear_bias_tables(ctypes.byref(d), 0.1, 0.1, None, P(FAKE),
                                       None) == hstu.HSTU_E_INVAL
    bad = _desc()
    bad.input_norm = 2
    assert _attn(lib, bad, _jag()) == hstu.HSTU_E_INVAL
    assert b"input_norm" in lib.hstu_last_error()
    n1 = _desc()
    n1.input_norm = 1
    base = lib.hstu_layer_workspace_size(ctypes.byref(d), ctypes.byref(_jag()))
    assert lib.hstu_layer_workspace_size(ctypes.byref(n1), ctypes.byref(_jag())) == base + 10240


def test_cache_concat_validates(lib):
    P = ctypes.c_void_p
    d = _desc()
    a = hstu.KVCache(FAKE, FAKE, FAKE, FAKE, 8, 10)
    n = hstu.KVCache(FAKE + 1024, FAKE + 2048, FAKE + 4096, FAKE + 8192, 8, 5)
    cc = lambda B, a_, n_, o, t, k, v: lib.hstu_kv_cache_concat(
        ctypes.byref(d), B, ctypes.byref(a_) if a_ else None, ctypes.byref(n_) if n_ else None,
        P(o), P(t), P(k), P(v), None)
    out = (FAKE + 65536, FAKE + 131072, FAKE + 262144, FAKE + 524288)
    assert cc(-1, a, n, *out) == hstu.HSTU_E_INVAL
    assert cc(2, None, n, *out) == hstu.HSTU_E_INVAL
    assert cc(0, a, n, *out) == hstu.HSTU_E_INVAL                  # rows without sequences
    assert cc(2, a, n, out[0], out[1], FAKE, out[3]) == hstu.HSTU_E_INVAL   # out_k aliases a.k
    assert cc(2, a, n, out[0], out[1], out[2] + 8, out[3]) == hstu.HSTU_E_INVAL   # misaligned
    bad = hstu.KVCache(FAKE, FAKE, FAKE, FAKE, 8, -1)
    assert cc(2, bad, n, *out) == hstu.HSTU_E_INVAL


def test_backward_validates(lib):
    """hstu_layer_bwd supports fp32 plain causal layers; everything else is
    refused on the host, before any launch."""
    P = ctypes.c_void_p
    f = hstu.make_desc(64, 2, hstu.HSTU_F32, 255)
    params = hstu.LayerParams(FAKE, None, FAKE, None, None, None, FAKE, FAKE)
    grads = hstu.LayerGrads(*([FAKE] * 8))
    jag = _jag()
    ws = lib.hstu_layer_bwd_workspace_size(ctypes.byref(f), ctypes.byref(jag))
    assert ws == 17 * 2560 + 256
    call = lambda desc, j=jag, g=grads, p=params, dx=FAKE + 4096, wsb=ws: lib.hstu_layer_bwd(
        ctypes.byref(desc), ctypes.byref(p) if p else None, ctypes.byref(j),
        P(FAKE), P(FAKE + 8192), P(dx), ctypes.byref(g) if g else None, P(FAKE), wsb, None)
    assert call(_desc()) == hstu.HSTU_E_UNSUPPORTED                 # bf16
    n1 = hstu.make_desc(64, 2, hstu.HSTU_F32, 255, input_norm=True)
    assert call(n1) == hstu.HSTU_E_INVAL                          # dln1_gamma/dln1_beta unset
    tj = hstu.Jagged(2, 6, 10, FAKE, FAKE, FAKE)                     # targets
    assert call(f, j=tj) == hstu.HSTU_E_UNSUPPORTED
    assert call(f, g=None) == hstu.HSTU_E_INVAL
    half = hstu.LayerGrads(*([FAKE] * 7 + [None]))
    assert call(f, g=half) == hstu.HSTU_E_INVAL
    assert call(f, p=None) == hstu.HSTU_E_INVAL
    assert call(f, dx=FAKE) == hstu.HSTU_E_INVAL                     # dx aliases x
    assert call(f, wsb=ws - 1) == hstu.HSTU_E_WORKSPACE
    # bf16 products: Xin and W1 as bf16 hi/lo splits (3 columns per value),
    # bf16 G, W2 (f2), dY, dZ (T x d, T x 4d),
    # the transposed dY, G, Xin (d x 32) and dZ (4d x 32) padded to one
    # 32-token split, W1^T, W2^T and one split's partial dW1, each rounded up
    # to 256 bytes
    g16 = hstu.make_desc(64, 2, hstu.HSTU_F32, 255, gemm_bwd_bf16=True)
    extra = (3 * 1280 + 3 * 32768 + 1280 + 8192) + 1280 + 5120 + 3 * 4096 + 16384 + 32768 + 8192 + 65536
    assert lib.hstu_layer_bwd_workspace_size(ctypes.byref(g16), ctypes.byref(jag)) == ws + extra
    assert call(g16) == hstu.HSTU_E_WORKSPACE
    bad = hstu.make_desc(64, 2, hstu.HSTU_F32, 255)
    bad.gemm_bwd_bf16 = 2
    assert call(bad) == hstu.HSTU_E_INVAL
    assert b"gemm_bwd_bf16" in lib.hstu_last_error()


def test_train_pair_validates(lib):
    """hstu_layer_fwd_train and hstu_layer_bwd_after_fwd take what
    hstu_layer_bwd takes, and refuse the same layers on the host."""
    P = ctypes.c_void_p
    f = hstu.make_desc(64, 2, hstu.HSTU_F32, 255)
    params = hstu.LayerParams(FAKE, None, FAKE, None, None, None, FAKE, FAKE)
    grads = hstu.LayerGrads(*([FAKE] * 8))
    jag = _jag()
    ws = lib.hstu_layer_bwd_workspace_size(ctypes.byref(f), ctypes.byref(jag))
    fwd = lambda desc, y=FAKE + 4096, wsb=ws, p=params: lib.hstu_layer_fwd_train(
        ctypes.byref(desc), ctypes.byref(p) if p else None, ctypes.byref(jag), P(FAKE), P(y), P(FAKE), wsb,
        None)
    assert fwd(_desc()) == hstu.HSTU_E_UNSUPPORTED                  # bf16
    assert fwd(f, y=FAKE) == hstu.HSTU_E_INVAL                       # y aliases x
    assert fwd(f, y=None) == hstu.HSTU_E_INVAL
    assert fwd(f, p=None) == hstu.HSTU_E_INVAL
    assert fwd(f, wsb=ws - 1) == hstu.HSTU_E_WORKSPACE
    bwd = lambda desc, g=grads, dx=FAKE + 4096: lib.hstu_layer_bwd_after_fwd(
        ctypes.byref(desc), ctypes.byref(params), ctypes.byref(jag), P(FAKE), P(FAKE + 8192), P(dx),
        ctypes.byref(g) if g else None, P(FAKE), ws, None)
    assert bwd(_desc()) == hstu.HSTU_E_UNSUPPORTED
    assert bwd(f, g=None) == hstu.HSTU_E_INVAL
    assert bwd(f, dx=FAKE) == hstu.HSTU_E_INVAL


def test_binding_raises_with_message(lib):
    with pytest.raises(hstu.HstuError) as e:
        hstu.hstu_attn_fwd(None, _jag(), None, None, None, None, None, None, None, None, stream=0)
    assert e.value.status == hstu.HSTU_E_INVAL


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "hstu_sequential_transducer_jagged_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_noalloc_rejects_a_work_list_larger_than_its_scratch(lib):
    """hstu_attn_fwd_noalloc: a batch whose work list alone exceeds the
    static scratch (100 000 sequences of up to 8192 tokens: 12.8 M work
    units) is refused with HSTU_E_WORKSPACE before anything is enqueued."""
    P = ctypes.c_void_p
    d = hstu.make_desc(512, 8, hstu.HSTU_BF16, 2 * 8192 - 1)
    jag = hstu.Jagged(100_000, 8192, 200_000, FAKE, FAKE, None)
    st = lib.hstu_attn_fwd_noalloc(ctypes.byref(d), ctypes.byref(jag), None, P(FAKE), P(FAKE), P(FAKE),
                                   P(FAKE), P(FAKE), P(FAKE), None)
    assert st == hstu.HSTU_E_WORKSPACE
    assert b"static scratch" in lib.hstu_last_error()


def test_bias_mode_and_token_type_validation(lib):
    """The type-aware rab and the in-kernel parameter-free bias: descriptor
    and pointer checks made on the host before any launch."""
    P = ctypes.c_void_p
    d = _desc()
    d.num_token_types = hstu.HSTU_MAX_TOKEN_TYPES + 1
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc()
    d.num_token_types = -1
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc()
    d.bias_mode = 2
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc()
    d.bias_mode = hstu.HSTU_BIAS_LINEAR
    d.linear_m_p = float("inf")
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    d = _desc()
    d.bias_mode = hstu.HSTU_BIAS_LINEAR
    d.num_token_types = 2
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_UNSUPPORTED
    # typed: token types must be given for own tokens and for a non-empty cache
    d = _desc()
    d.num_token_types = 3
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    assert b"token_types" in lib.hstu_last_error()
    j = _jag()
    j.token_types = FAKE
    cache = hstu.KVCache(FAKE, FAKE, FAKE, FAKE, 8, 100)
    d.pos_table_len = 255
    assert _attn(lib, d, j, cache) == hstu.HSTU_E_INVAL
    assert b"cache token_types" in lib.hstu_last_error()
    # the parameter-free bias reads no tables and no position bound applies
    d = _desc(pos_table_len=3)
    d.bias_mode = hstu.HSTU_BIAS_LINEAR
    st = lib.hstu_attn_fwd(ctypes.byref(d), ctypes.byref(_jag(B=0, T=0, mx=0)), None, P(FAKE),
                           P(FAKE), P(FAKE), None, None, P(FAKE), None, 0, None)
    assert st == hstu.HSTU_OK
    d = _desc(pos_table_len=3)                                 # tables: n_max 2 < 6
    assert _attn(lib, d, _jag()) == hstu.HSTU_E_INVAL
    # the backward pass takes the untyped table bias only
    f = hstu.make_desc(64, 1, hstu.HSTU_F32, 255, num_token_types=2)
    params = hstu.LayerParams(*([FAKE] * 8))
    grads = hstu.LayerGrads(*([FAKE] * 10))
    j = _jag()
    j.token_types = FAKE
    assert lib.hstu_layer_bwd(ctypes.byref(f), ctypes.byref(params), ctypes.byref(j), P(FAKE),
                              P(FAKE), P(FAKE + 4096), ctypes.byref(grads), P(FAKE), 1 << 30,
                              None) == hstu.HSTU_E_UNSUPPORTED
    assert b"untyped table bias" in lib.hstu_last_error()


PROBE_HEADER = os.path.join(ROOT, "include", "hstu_probe.h")


def test_probe_library_exports_its_header():
    from hstu_sequential_transducer_jagged_amd import probe
    text = open(PROBE_HEADER).read()
    declared = sorted(set(re.findall(r"^\s*int\s*(hstu_probe_\w+)\s*\(", text, re.MULTILINE)))
    assert declared == sorted(probe.EXPORTS)
    if not os.path.exists(probe.LIB_PATH):
        from hstu_sequential_transducer_jagged_amd import build
        build.build()
    lib = probe.load()
    for name in declared:
        assert hasattr(lib, name), name
    # invalid arguments are refused before any launch (hipErrorInvalidValue = 1)
    assert lib.hstu_probe_copy(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 8), 16, None) == 1
    assert lib.hstu_probe_copy(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64), 24, None) == 1
    assert lib.hstu_probe_mfma_bf16(0, 1, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == 1
