"""Thin ctypes binding of libcad.so (argument marshalling only).

Every function here forwards device pointers of torch tensors to the C ABI declared in
include/cad.h and raises on a non-zero status.  All arithmetic runs in the library's HIP
kernels; there is no fallback path: if libcad.so is missing or fails to load, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcad.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "cad.h")

CAD_OK, CAD_EINVAL, CAD_EUNSUPPORTED, CAD_ECAPACITY, CAD_EHIP, CAD_EWORKSPACE = 0, -1, -2, -3, -4, -5
DTYPE_BF16, DTYPE_F32 = 0, 1
MASK_CAUSAL, MASK_BLOCK = 0, 1
COMMIT_ALL, KV_ONLY, LOGITS_LAST = 1, 2, 4
MAX_ALLOWED = 16


class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int), ("vocab", ctypes.c_int),
                ("dtype", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_double),
                ("embed", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p), ("w_lm", ctypes.c_void_p)]


class KVDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("err", ctypes.c_void_p), ("B", ctypes.c_int), ("cap", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("dtype", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcad.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m spec_verify_cad_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.cad_ngram_lookup.argtypes = [vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    L.cad_ngram_lookup.restype = i32
    L.cad_ngram_lookup_longest.argtypes = [vp, i64, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.cad_ngram_lookup_longest.restype = i32
    L.cad_span_forward.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(KVDesc), vp, i32, i32, i32, i32, i32,
                                   i32, vp, vp, vp, vp, vp, sz, vp]
    L.cad_span_forward.restype = i32
    L.cad_stack_span_forward.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(KVDesc), vp, i32, i32, i32,
                                         i32, i32, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.cad_stack_span_forward.restype = i32
    L.cad_span_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(KVDesc), vp, i32, i32, i32, i32,
                                           i32, i32, vp, vp, vp, vp, vp]
    L.cad_span_forward_noalloc.restype = i32
    L.cad_stack_span_forward_allowed.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(KVDesc), vp, i32, i32,
                                                 i32, vp, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.cad_stack_span_forward_allowed.restype = i32
    L.cad_stack_span_forward_sampled.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(KVDesc), vp, i32, i32,
                                                 i32, ctypes.c_float, ctypes.c_uint64, vp, vp, vp, vp, vp,
                                                 ctypes.c_size_t, vp]
    L.cad_stack_span_forward_sampled.restype = i32
    L.cad_stack_span_forward_workspace.argtypes = [ctypes.POINTER(LayerDesc), i32, i32, i32, i32, i32, i32, i32, i32]
    L.cad_stack_span_forward_workspace.restype = ctypes.c_size_t
    L.cad_span_forward_sampled.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(KVDesc), vp, i32, i32, i32,
                                           ctypes.c_float, ctypes.c_uint64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.cad_span_forward_sampled.restype = i32
    L.cad_span_forward_allowed.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(KVDesc), vp, i32, i32, i32, vp,
                                           i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.cad_span_forward_allowed.restype = i32
    L.cad_span_forward_workspace.argtypes = [ctypes.POINTER(LayerDesc), i32, i32, i32, i32, i32, i32, i32]
    L.cad_span_forward_workspace.restype = sz
    L.cad_accept_scan.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp, i32,
                                  ctypes.POINTER(KVDesc), vp]
    L.cad_accept_scan.restype = i32
    L.cad_stack_accept_scan.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp, i32,
                                        ctypes.POINTER(KVDesc), i32, vp]
    L.cad_stack_accept_scan.restype = i32
    L.cad_status_string.argtypes = [i32]
    L.cad_status_string.restype = ctypes.c_char_p
    L.cad_version.restype = i32
    L.cad_profile_enable.argtypes = [i32]
    L.cad_profile_enable.restype = i32
    L.cad_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    L.cad_profile_read.restype = i32
    L.cad_profile_stage_name.argtypes = [i32]
    L.cad_profile_stage_name.restype = ctypes.c_char_p
    _lib = L
    return L


def header_functions() -> list:
    """Names of the functions include/cad.h declares."""
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(cad_[a-z_]+)\s*\(", src, re.M)))


class CadError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib().cad_status_string(status).decode()} ({status})")
        self.status = status


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != CAD_OK:
        raise CadError(status, what)


# ---------------------------------------------------------------------------------------
# device-resident layer and cache (plain tensors + the descriptors pointing at them)
# ---------------------------------------------------------------------------------------

class DeviceLayer:
    """Weights of one layer on the GPU and the cad_layer_desc that points at them."""

    def __init__(self, shape, weights: dict, device="cuda"):
        import torch
        self.shape = shape
        self.t = {}
        for name, arr in weights.items():
            if arr.dtype == np.uint16:
                t = torch.from_numpy(arr.view(np.int16)).to(device)
            else:
                t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
            self.t[name] = t
        self.desc = self.make_desc()

    @classmethod
    def from_tensors(cls, shape, tensors: dict) -> "DeviceLayer":
        """A layer over device tensors the caller already holds (bf16 as int16 bit patterns)."""
        self = cls.__new__(cls)
        self.shape, self.t = shape, dict(tensors)
        self.desc = self.make_desc()
        return self

    def make_desc(self, **override) -> LayerDesc:
        s = self.shape
        t = dict(self.t, **override)
        return LayerDesc(s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                         DTYPE_BF16 if s.dtype == "bf16" else DTYPE_F32, s.rms_eps, s.rope_base,
                         *(t[n].data_ptr() if n in t else None
                           for n in ("embed", "w_qkv", "w_o", "w_gate_up", "w_down", "w_lm")))


class DeviceCache:
    """KV cache of B sequences: k [B, Hkv, cap, d], v [B, Hkv, d, cap] (dim-major), len [B], err [B].

    `len_tensor` may supply the int32 [B] length tensor (e.g. a view of a larger one, so the
    lengths of several caches can be reset by one fill)."""

    def __init__(self, shape, B: int, cap: int, device="cuda", len_tensor=None):
        import torch
        dt = torch.int16 if shape.dtype == "bf16" else torch.float32
        self.shape, self.B, self.cap = shape, B, cap
        self.k = torch.zeros((B, shape.n_kv_heads, cap, shape.head_dim), dtype=dt, device=device)
        self.v = torch.zeros((B, shape.n_kv_heads, shape.head_dim, cap), dtype=dt, device=device)
        self.len = torch.zeros(B, dtype=torch.int32, device=device) if len_tensor is None else len_tensor
        assert self.len.dtype == torch.int32 and self.len.numel() == B and self.len.is_contiguous()
        self.err = torch.zeros(B, dtype=torch.int32, device=device)
        self.desc = KVDesc(self.k.data_ptr(), self.v.data_ptr(), self.len.data_ptr(), self.err.data_ptr(), B, cap,
                           shape.n_kv_heads, shape.head_dim, DTYPE_BF16 if shape.dtype == "bf16" else DTYPE_F32)


class DeviceStack:
    """A stack of layers of one shape: the embedding of the first and the LM head of the last
    are used.  `descs` is the descriptor array the stack call takes."""

    def __init__(self, layers: list):
        self.layers = list(layers)
        self.shape = self.layers[0].shape
        self.n = len(self.layers)
        self.descs = (LayerDesc * self.n)(*[l.desc for l in self.layers])


class StackCache:
    """One KV cache per layer of a stack, all sharing one length tensor (and layer 0's error
    flags, which the stack call uses)."""

    def __init__(self, shape, n_layers: int, B: int, cap: int, device="cuda"):
        import torch
        self.shape, self.B, self.cap, self.n = shape, B, cap, n_layers
        self.len = torch.zeros(B, dtype=torch.int32, device=device)
        self.caches = [DeviceCache(shape, B, cap, device=device, len_tensor=self.len) for _ in range(n_layers)]
        self.err = self.caches[0].err
        self.descs = (KVDesc * n_layers)(*[c.desc for c in self.caches])


# ---------------------------------------------------------------------------------------
# the three calls
# ---------------------------------------------------------------------------------------

def _row_stride(t) -> int:
    """Elements between rows of a [B, stride] history (a single row may carry any stride)."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def ngram_lookup(ctx, ctx_len, n: int, W: int, D: int, with_current: int, draft, draft_len, match_pos=None,
                 stream=None):
    B = ctx.shape[0]
    _check(lib().cad_ngram_lookup(_ptr(ctx), _row_stride(ctx), _ptr(ctx_len), B, n, W, D, with_current, _ptr(draft),
                                  _ptr(draft_len), _ptr(match_pos), _stream(stream)), "cad_ngram_lookup")


def ngram_lookup_longest(ctx, ctx_len, n_max: int, n_min: int, W: int, D: int, with_current: int, draft, draft_len,
                         match_pos=None, match_n=None, stream=None):
    B = ctx.shape[0]
    _check(lib().cad_ngram_lookup_longest(_ptr(ctx), _row_stride(ctx), _ptr(ctx_len), B, n_max, n_min, W, D,
                                          with_current, _ptr(draft), _ptr(draft_len), _ptr(match_pos), _ptr(match_n),
                                          _stream(stream)), "cad_ngram_lookup_longest")


def span_forward_workspace(layer: DeviceLayer, B: int, Nq: int, mode: int = MASK_CAUSAL, W: int = 1, D: int = 1,
                           cap: int = 1, flags: int = 0) -> int:
    return lib().cad_span_forward_workspace(ctypes.byref(layer.desc), B, Nq, mode, W, D, cap, flags)


def alloc_workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def span_forward(layer: DeviceLayer, cache: DeviceCache, tokens, Nq: int, mode: int = MASK_CAUSAL, W: int = 1,
                 D: int = 1, flags: int = 0, argmax_out=None, hidden_out=None, logits_out=None, workspace=None,
                 stream=None, top2_gap=None):
    B = cache.B
    if workspace is None:
        workspace = alloc_workspace(span_forward_workspace(layer, B, Nq, mode, W, D, cache.cap, flags))
    _check(lib().cad_span_forward(ctypes.byref(layer.desc), ctypes.byref(cache.desc), _ptr(tokens), B, Nq, mode, W, D,
                                  flags, _ptr(argmax_out), _ptr(hidden_out), _ptr(logits_out), _ptr(top2_gap),
                                  _ptr(workspace), workspace.numel(), _stream(stream)), "cad_span_forward")
    return workspace


NOALLOC_SCRATCH_BYTES = 32 << 20


def span_forward_noalloc(layer: DeviceLayer, cache: DeviceCache, tokens, Nq: int, mode: int = MASK_CAUSAL, W: int = 1,
                         D: int = 1, flags: int = 0, argmax_out=None, hidden_out=None, logits_out=None, top2_gap=None,
                         stream=None):
    """cad_span_forward with the library's static device workspace (for callers that cannot
    allocate, e.g. under graph capture); forwards needing more than 32 MiB of workspace raise."""
    _check(lib().cad_span_forward_noalloc(ctypes.byref(layer.desc), ctypes.byref(cache.desc), _ptr(tokens), cache.B,
                                          Nq, mode, W, D, flags, _ptr(argmax_out), _ptr(hidden_out),
                                          _ptr(logits_out), _ptr(top2_gap), _stream(stream)),
           "cad_span_forward_noalloc")


def stack_span_forward_workspace(stack: DeviceStack, B: int, Nq: int, mode: int = MASK_CAUSAL, W: int = 1,
                                 D: int = 1, cap: int = 0, flags: int = 0) -> int:
    n = lib().cad_stack_span_forward_workspace(stack.descs, stack.n, B, Nq, mode, W, D, cap, flags)
    if n == 0:
        raise CadError(CAD_EINVAL, "cad_stack_span_forward_workspace")
    return n


def stack_span_forward(stack: DeviceStack, cache: StackCache, tokens, Nq: int, mode: int = MASK_CAUSAL, W: int = 1,
                       D: int = 1, flags: int = 0, argmax_out=None, hidden_out=None, logits_out=None,
                       workspace=None, stream=None, top2_gap=None):
    if cache.n != stack.n:
        raise ValueError("one cache per layer")
    B = cache.B
    if workspace is None:
        workspace = alloc_workspace(stack_span_forward_workspace(stack, B, Nq, mode, W, D, cache.cap, flags))
    _check(lib().cad_stack_span_forward(stack.descs, stack.n, cache.descs, _ptr(tokens), B, Nq, mode, W, D, flags,
                                        _ptr(argmax_out), _ptr(hidden_out), _ptr(logits_out), _ptr(top2_gap),
                                        _ptr(workspace), workspace.numel(), _stream(stream)), "cad_stack_span_forward")
    return workspace


def stack_span_forward_allowed(stack: DeviceStack, cache: StackCache, tokens, Nq: int, allowed, A: int,
                               flags: int = 0, argmax_out=None, logits_out=None, hidden_out=None, workspace=None,
                               stream=None):
    if cache.n != stack.n:
        raise ValueError("one cache per layer")
    B = cache.B
    if workspace is None:
        workspace = alloc_workspace(stack_span_forward_workspace(stack, B, Nq, MASK_CAUSAL, 1, 1, cache.cap, flags))
    _check(lib().cad_stack_span_forward_allowed(stack.descs, stack.n, cache.descs, _ptr(tokens), B, Nq, flags,
                                                _ptr(allowed), A, _ptr(argmax_out), _ptr(logits_out),
                                                _ptr(hidden_out), _ptr(workspace), workspace.numel(),
                                                _stream(stream)), "cad_stack_span_forward_allowed")
    return workspace


def stack_span_forward_sampled(stack: DeviceStack, cache: StackCache, tokens, Nq: int, temperature: float, seed: int,
                               draft_len=None, flags: int = 0, pred_out=None, logits_out=None, hidden_out=None,
                               workspace=None, stream=None):
    if cache.n != stack.n:
        raise ValueError("one cache per layer")
    B = cache.B
    if workspace is None:
        workspace = alloc_workspace(stack_span_forward_workspace(stack, B, Nq, MASK_CAUSAL, 1, 1, cache.cap, flags))
    _check(lib().cad_stack_span_forward_sampled(stack.descs, stack.n, cache.descs, _ptr(tokens), B, Nq, flags,
                                                float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(draft_len),
                                                _ptr(pred_out), _ptr(logits_out), _ptr(hidden_out), _ptr(workspace),
                                                workspace.numel(), _stream(stream)), "cad_stack_span_forward_sampled")
    return workspace


def span_forward_sampled(layer: DeviceLayer, cache: DeviceCache, tokens, Nq: int, temperature: float, seed: int,
                         draft_len=None, flags: int = 0, pred_out=None, logits_out=None, hidden_out=None,
                         workspace=None, stream=None):
    """Causal span forward whose LM head draws (stochastic verification of the drafts in
    tokens[:, 1:], draft_len [B] per sequence, or plain draws when draft_len is None)."""
    B = cache.B
    if workspace is None:
        workspace = alloc_workspace(span_forward_workspace(layer, B, Nq, MASK_CAUSAL, 1, 1, cache.cap, flags))
    _check(lib().cad_span_forward_sampled(ctypes.byref(layer.desc), ctypes.byref(cache.desc), _ptr(tokens), B, Nq,
                                          flags, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(draft_len),
                                          _ptr(pred_out), _ptr(logits_out), _ptr(hidden_out), _ptr(workspace),
                                          workspace.numel(), _stream(stream)), "cad_span_forward_sampled")
    return workspace


def span_forward_allowed(layer: DeviceLayer, cache: DeviceCache, tokens, Nq: int, allowed, A: int, flags: int = 0,
                         argmax_out=None, logits_out=None, hidden_out=None, workspace=None, stream=None):
    """Causal span forward with the argmax restricted to each row's A allowed ids (int32 [B*Nq, A])."""
    B = cache.B
    if workspace is None:
        workspace = alloc_workspace(span_forward_workspace(layer, B, Nq, MASK_CAUSAL, 1, 1, cache.cap, flags))
    _check(lib().cad_span_forward_allowed(ctypes.byref(layer.desc), ctypes.byref(cache.desc), _ptr(tokens), B, Nq,
                                          flags, _ptr(allowed), A, _ptr(argmax_out), _ptr(logits_out),
                                          _ptr(hidden_out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "cad_span_forward_allowed")
    return workspace


def accept_scan(draft, with_current: int, draft_len, pred, first_pred, B: int, W: int, D: int, mode: int,
                accepted, best_w, emitted, n_emitted, ctx=None, ctx_len=None, ctx_cap: int = 0,
                cache: DeviceCache | None = None, stream=None):
    kvp = ctypes.byref(cache.desc) if cache is not None else None
    _check(lib().cad_accept_scan(_ptr(draft), with_current, _ptr(draft_len), _ptr(pred), _ptr(first_pred), B, W, D,
                                 mode, _ptr(accepted), _ptr(best_w), _ptr(emitted), _ptr(n_emitted), _ptr(ctx),
                                 _row_stride(ctx) if ctx is not None else 0, _ptr(ctx_len), ctx_cap, kvp,
                                 _stream(stream)), "cad_accept_scan")


def stack_accept_scan(draft, with_current: int, draft_len, pred, first_pred, B: int, W: int, D: int, mode: int,
                      accepted, best_w, emitted, n_emitted, cache: StackCache, ctx=None, ctx_len=None,
                      ctx_cap: int = 0, stream=None):
    """Accept scan after a verify forward through a stack: in block mode the winner's rows move in
    every layer's cache."""
    _check(lib().cad_stack_accept_scan(_ptr(draft), with_current, _ptr(draft_len), _ptr(pred), _ptr(first_pred), B, W,
                                       D, mode, _ptr(accepted), _ptr(best_w), _ptr(emitted), _ptr(n_emitted),
                                       _ptr(ctx), _row_stride(ctx) if ctx is not None else 0, _ptr(ctx_len), ctx_cap,
                                       cache.descs, cache.n, _stream(stream)), "cad_stack_accept_scan")


# ---------------------------------------------------------------------------------------
# diagnostics
# ---------------------------------------------------------------------------------------

def profile_enable(on: bool = True):
    _check(lib().cad_profile_enable(1 if on else 0), "cad_profile_enable")


def profile_read() -> dict:
    """Per-stage (total ms, launches) recorded since the last read; waits for the events."""
    n = 32
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    st = lib().cad_profile_read(n, ms, cnt)
    if st < 0:
        raise CadError(st, "cad_profile_read")
    return {lib().cad_profile_stage_name(i).decode(): (ms[i], cnt[i]) for i in range(st) if cnt[i]}
