"""An ideal fp32-accumulating forward of the layer (test-side reference for the error budget).

The oracle accumulates in fp64.  Any GPU forward accumulates in fp32, rounds to bf16 at the same
eight points, and therefore drifts from the oracle wherever an fp32 sum lands within its own
rounding error of a bf16 rounding boundary; the differences cascade through the following norms
and projections.  This module is the same arithmetic as the oracle with every product, reduction
and softmax in float32 (numpy), so its distance to the oracle on the same inputs is the drift
that fp32 accumulation alone causes.  The full-size GPU parity tests bound the GPU's distance to
the oracle by a small multiple of this one.  It shares no code with the HIP library; it reads the
oracle's layer weights (fp64 copies of the stored values) and uses the oracle's bf16 rounding.
"""
from __future__ import annotations

import numpy as np

import oracle as O

f32 = np.float32


def _w(L, name):
    """float32 copy of one weight of an oracle layer (kept on the layer object)."""
    cache = L.__dict__.setdefault("_ideal_f32", {})
    if name not in cache:
        cache[name] = np.ascontiguousarray(getattr(L, name).astype(f32))
    return cache[name]


def release(L):
    """Drop the float32 weight copies of a layer."""
    L.__dict__.pop("_ideal_f32", None)


def _rnd(L, a):
    a = np.asarray(a, dtype=f32)
    return O.round_bf16(a.astype(np.float64)).astype(f32) if L.precision == "bf16" else a


def _rms(L, v):
    v = np.asarray(v, dtype=f32)
    return (v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True, dtype=f32) + f32(L.eps))).astype(f32)


def _proj(a, w):
    return (a @ w.T).astype(f32)


class Cache:
    def __init__(self, L, cap: int):
        self.K = np.zeros((L.n_kv_heads, cap, L.head_dim), f32)
        self.V = np.zeros((L.n_kv_heads, cap, L.head_dim), f32)
        self.length = 0
        self.cap = cap

    def copy(self):
        c = Cache.__new__(Cache)
        c.K, c.V, c.length, c.cap = self.K.copy(), self.V.copy(), self.length, self.cap
        return c


def _rope(L, t, pos):
    d, half = L.head_dim, L.head_dim // 2
    c, s = O.rope_cos_sin(np.asarray(pos), d, L.rope_base)
    c, s = c.astype(f32)[:, None, :], s.astype(f32)[:, None, :]
    return np.concatenate([t[..., :half] * c - t[..., half:] * s, t[..., half:] * c + t[..., :half] * s], -1)


def _kv(L, u, pos):
    n, d = u.shape[0], L.head_dim
    k = _proj(u, _w(L, "wk")).reshape(n, L.n_kv_heads, d)
    v = _proj(u, _w(L, "wv")).reshape(n, L.n_kv_heads, d)
    return _rnd(L, _rope(L, k, pos)), _rnd(L, v)


def cache_from_tokens(L, tokens, cap: int, chunk: int = 4096) -> Cache:
    """Cache rows of a token prefix through one layer (its K/V depend on the token only)."""
    tokens = np.asarray(tokens)
    c = Cache(L, cap)
    for s in range(0, len(tokens), chunk):
        t = tokens[s:s + chunk]
        u = _rnd(L, _rms(L, _w(L, "embed")[t]))
        k, v = _kv(L, u, np.arange(s, s + len(t)))
        c.K[:, s:s + len(t)] = k.transpose(1, 0, 2)
        c.V[:, s:s + len(t)] = v.transpose(1, 0, 2)
    c.length = len(tokens)
    return c


def _attend(L, cache, u, pos, slots, mask):
    n, d = u.shape[0], L.head_dim
    q = _rnd(L, _rope(L, _proj(u, _w(L, "wq")).reshape(n, L.n_q_heads, d), pos))
    k, v = _kv(L, u, pos)
    cache.K[:, slots] = k.transpose(1, 0, 2)
    cache.V[:, slots] = v.transpose(1, 0, 2)
    S = mask.shape[1]
    o = np.zeros((n, L.n_q_heads, d), f32)
    for h in range(L.n_q_heads):
        g = h // (L.n_q_heads // L.n_kv_heads)
        sc = np.where(mask, (q[:, h] @ cache.K[g, :S].T) / f32(np.sqrt(d)), -np.inf).astype(f32)
        p = np.exp(sc - sc.max(-1, keepdims=True)).astype(f32)
        o[:, h] = (p @ cache.V[g, :S]) / p.sum(-1, keepdims=True)
    return _rnd(L, o.reshape(n, -1))


def _block(L, x, o):
    h1 = (x + _proj(o, _w(L, "wo"))).astype(f32)
    u2 = _rnd(L, _rms(L, h1))
    gt, ut = _proj(u2, _w(L, "wg")), _proj(u2, _w(L, "wu"))
    act = _rnd(L, gt / (1 + np.exp(-gt)) * ut)
    h2 = (h1 + _proj(act, _w(L, "wd"))).astype(f32)
    return h2, _rnd(L, _rms(L, h2))


def _head(L, u3, h2):
    logits = _proj(u3, _w(L, "wlm")).astype(np.float64)
    return {"hidden_out": _rnd(L, h2).astype(np.float64), "logits": logits,
            "argmax": np.argmax(logits, axis=-1)}


def stack_span_forward(layers, caches, tokens, mode="causal", W=1, D=0, commit=True) -> dict:
    """The oracle's stack span forward (append-then-attend, explicit mask) in float32."""
    tokens = np.asarray(tokens)
    n, base = len(tokens), caches[0].length
    slots, pos, mask = O.span_layout(base, n, mode, W, D)
    x = _w(layers[0], "embed")[tokens]
    u = _rnd(layers[0], _rms(layers[0], x))
    for L, c in zip(layers, caches):
        o = _attend(L, c, u, pos, slots, mask)
        x, u = _block(L, x, o)
    if commit:
        for c in caches:
            c.length = base + n
    return _head(layers[-1], u, x)


def span_forward(L, cache, tokens, mode="causal", W=1, D=0, commit=True) -> dict:
    return stack_span_forward([L], [cache], tokens, mode, W, D, commit)


def stack_prefill(layers, tokens, cap: int, chunk: int = 512) -> list:
    caches = [Cache(L, cap) for L in layers]
    tokens = np.asarray(tokens)
    for s in range(0, len(tokens), chunk):
        t = tokens[s:s + chunk]
        n, base = len(t), caches[0].length
        slots, pos, mask = O.span_layout(base, n, "causal")
        x = _w(layers[0], "embed")[t]
        u = _rnd(layers[0], _rms(layers[0], x))
        for L, c in zip(layers, caches):
            o = _attend(L, c, u, pos, slots, mask)
            x, u = _block(L, x, o)
        for c in caches:
            c.length = base + n
    return caches
