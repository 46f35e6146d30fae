"""The C-ABI library loads and exports every function include/cad.h declares; host-side
argument checks reject bad calls before anything is enqueued (no GPU needed)."""
import ctypes

import pytest

from spec_verify_cad_amd import cad


def test_header_declares_the_three_calls():
    names = cad.header_functions()
    for n in ("cad_ngram_lookup", "cad_span_forward", "cad_accept_scan", "cad_span_forward_workspace",
              "cad_span_forward_allowed", "cad_ngram_lookup_longest", "cad_status_string", "cad_version",
              "cad_stack_accept_scan"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = cad.lib()
    for n in cad.header_functions():
        assert hasattr(L, n), n
    assert L.cad_version() >= 100
    assert L.cad_status_string(cad.CAD_EWORKSPACE).decode() == "workspace missing or too small"


def _desc(**kw):
    d = cad.LayerDesc(256, 4, 4, 64, 1024, 1024, cad.DTYPE_BF16, 1e-6, 1e4, 1, 1, 1, 1, 1, 1)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_query_and_invalid_shapes():
    L = cad.lib()
    d = _desc()
    full = L.cad_span_forward_workspace(ctypes.byref(d), 1, 8, 0, 1, 1, 160, 0)
    kvo = L.cad_span_forward_workspace(ctypes.byref(d), 1, 8, 0, 1, 1, 160, cad.KV_ONLY)
    assert full > kvo > 0
    assert L.cad_span_forward_workspace(ctypes.byref(d), 1, 8, cad.MASK_BLOCK, 3, 3, 160, 0) == 0   # 3*3 != 8
    assert L.cad_span_forward_workspace(ctypes.byref(_desc(dtype=7)), 1, 8, 0, 1, 1, 160, 0) == 0
    assert L.cad_span_forward_workspace(None, 1, 8, 0, 1, 1, 160, 0) == 0


def test_host_argument_errors_return_before_launch():
    L = cad.lib()
    d = _desc()
    kv = cad.KVDesc(1, 1, 1, 1, 1, 160, 4, 64, cad.DTYPE_BF16)
    tok = ctypes.c_void_p(1)
    # null layer / tokens
    assert L.cad_span_forward(None, ctypes.byref(kv), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(kv), None, 1, 8, 0, 1, 1, 0, tok, None, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    # cache geometry that does not match the layer
    bad = cad.KVDesc(1, 1, 1, 1, 1, 160, 2, 64, cad.DTYPE_BF16)
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(bad), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    # unsupported head_dim
    d2 = _desc(head_dim=48)
    kv2 = cad.KVDesc(1, 1, 1, 1, 1, 160, 4, 48, cad.DTYPE_BF16)
    assert L.cad_span_forward(ctypes.byref(d2), ctypes.byref(kv2), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, tok, 1 << 30, None) == cad.CAD_EUNSUPPORTED
    # one head's K cache of 2 GiB or more (the tiled attention addresses it with 32-bit offsets)
    huge = cad.KVDesc(1, 1, 1, 1, 1, 1 << 24, 4, 64, cad.DTYPE_BF16)
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(huge), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, tok, 1 << 30, None) == cad.CAD_EUNSUPPORTED
    ok_cap = cad.KVDesc(1, 1, 1, 1, 1, (1 << 24) - 4, 4, 64, cad.DTYPE_BF16)
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(ok_cap), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, ctypes.c_void_p(8), 1 << 30, None) == cad.CAD_EWORKSPACE
    # workspace too small / misaligned
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(kv), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, ctypes.c_void_p(256), 16, None) == cad.CAD_EWORKSPACE
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(kv), tok, 1, 8, 0, 1, 1, 0, tok, None, None, None, ctypes.c_void_p(8), 1 << 30, None) == cad.CAD_EWORKSPACE
    # unknown flag, missing argmax output
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(kv), tok, 1, 8, 0, 1, 1, 8, tok, None, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    assert L.cad_span_forward(ctypes.byref(d), ctypes.byref(kv), tok, 1, 8, 0, 1, 1, 0, None, None, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    # grammar-masked forward: null set / output, set size, flags it does not take
    fa = L.cad_span_forward_allowed
    assert fa(ctypes.byref(d), ctypes.byref(kv), tok, 1, 1, 0, None, 4, tok, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    assert fa(ctypes.byref(d), ctypes.byref(kv), tok, 1, 1, 0, tok, 4, None, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    assert fa(ctypes.byref(d), ctypes.byref(kv), tok, 1, 1, 0, tok, 0, tok, None, None, tok, 1 << 30, None) == cad.CAD_EUNSUPPORTED
    assert fa(ctypes.byref(d), ctypes.byref(kv), tok, 1, 1, 0, tok, cad.MAX_ALLOWED + 1, tok, None, None, tok, 1 << 30,
              None) == cad.CAD_EUNSUPPORTED
    assert fa(ctypes.byref(d), ctypes.byref(kv), tok, 1, 1, cad.KV_ONLY, tok, 4, tok, None, None, tok, 1 << 30,
              None) == cad.CAD_EINVAL
    assert fa(ctypes.byref(d), ctypes.byref(kv), None, 1, 1, 0, tok, 4, tok, None, None, tok, 1 << 30, None) == cad.CAD_EINVAL
    # lookup / accept argument errors
    assert L.cad_ngram_lookup(tok, 16, tok, 1, 0, 1, 4, 0, tok, tok, None, None) == cad.CAD_EINVAL
    assert L.cad_ngram_lookup(tok, 16, tok, 1, 3, 9, 4, 0, tok, tok, None, None) == cad.CAD_EUNSUPPORTED
    assert L.cad_ngram_lookup(tok, 16, tok, 1, 3, 1, 65, 0, tok, tok, None, None) == cad.CAD_EUNSUPPORTED
    assert L.cad_accept_scan(tok, 1, tok, tok, None, 1, 2, 4, cad.MASK_CAUSAL, tok, None, tok, tok, None, 0, None, 0, None, None) == cad.CAD_EINVAL
    assert L.cad_accept_scan(tok, 0, tok, tok, None, 1, 2, 4, cad.MASK_BLOCK, tok, None, tok, tok, None, 0, None, 0, None, None) == cad.CAD_EINVAL
    # stack accept: no caches, no layers, block mode through several layers without best_w,
    # caches of another geometry
    sa = L.cad_stack_accept_scan
    kvs = (cad.KVDesc * 2)(cad.KVDesc(1, 1, 1, 1, 1, 160, 4, 64, cad.DTYPE_BF16),
                           cad.KVDesc(1, 1, 1, 1, 1, 160, 4, 64, cad.DTYPE_BF16))
    assert sa(tok, 0, tok, tok, tok, 1, 2, 4, cad.MASK_BLOCK, tok, tok, tok, tok, None, 0, None, 0, None, 2,
              None) == cad.CAD_EINVAL
    assert sa(tok, 0, tok, tok, tok, 1, 2, 4, cad.MASK_BLOCK, tok, tok, tok, tok, None, 0, None, 0, kvs, 0,
              None) == cad.CAD_EINVAL
    assert sa(tok, 0, tok, tok, tok, 1, 2, 4, cad.MASK_BLOCK, tok, None, tok, tok, None, 0, None, 0, kvs, 2,
              None) == cad.CAD_EINVAL
    kvs[1].head_dim = 32
    assert sa(tok, 0, tok, tok, tok, 1, 2, 4, cad.MASK_BLOCK, tok, tok, tok, tok, None, 0, None, 0, kvs, 2,
              None) == cad.CAD_EINVAL
    kvs[1].head_dim = 64
    assert sa(tok, 1, tok, tok, None, 1, 2, 4, cad.MASK_CAUSAL, tok, None, tok, tok, None, 0, None, 0, kvs, 2,
              None) == cad.CAD_EINVAL                            # causal mode takes W = 1
