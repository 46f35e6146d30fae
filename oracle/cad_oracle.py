"""Plain fp64 CPU oracle of the span-commit / verify path (test infrastructure only).

What is computed, and where the pages fix it
--------------------------------------------
* Copy-as-Decode, §2.4 "Copy-Span Splicing via Parallel Prefill": a copy span of N known
  tokens is appended to the KV cache by ONE ordinary prefill forward over the N tokens
  (self-attention and feed-forward over all N), instead of N decode forwards.
* Copy-as-Decode, Appendix K (position correctness): that forward advances the position
  ids by N exactly as N sequential decode steps would, RoPE being indexed by absolute
  position.  So the span forward must reproduce N single-token decode steps.  This oracle
  implements both (`decode_one` with a growing cache, `span_forward` with an explicit
  mask matrix) so the two can be compared.
* PLD page, "The n-gram match, precisely": the draft is the k tokens that followed an
  earlier occurrence of the last n tokens; most-recent match preferred; no match, no
  draft (`ngram_lookup`).
* PLD page, "Verification in a single parallel pass": left-to-right acceptance, a agreed
  draft tokens plus one bonus token from the target (`accept_causal`).
* SwitchSD page, block-triangular verification paragraph: W candidates concatenated after
  the anchor; candidate w sees the whole prefix and its own earlier tokens only; the
  longest validated continuation wins (`span_forward(mode="block")`, `accept_block`).

Readings where the pages are silent (all stated again in the design notes):
* the layer is a pre-norm Qwen2-style decoder layer: RMSNorm (gamma = 1) -> QKV ->
  half-split RoPE -> grouped-query attention -> O -> residual -> RMSNorm -> SwiGLU ->
  residual, then a final RMSNorm and an untied LM head; no biases;
* rounding points: activations are rounded to the layer's storage precision (bf16 with
  round-to-nearest-even, or fp32 for an fp32 layer) at R1 (normed input), R2/R3 (rotated
  q, rotated k and v as stored in the cache), R4 (attention output), R5 (second normed
  input), R6 (SwiGLU product), R7 (hidden output), R8 (final normed input); the residual
  stream and the logits are rounded to fp32; everything between is fp64;
* append-then-attend: all rows of a forward write their K/V first, and every query then
  reads keys as stored (rounded), its own included;
* argmax ties go to the lowest token id.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------------------

_EXP_BITS_DROPPED = 45          # fp64 keeps 52 fraction bits, bf16 keeps 7
_HALF_MINUS_ONE = np.uint64((1 << 44) - 1)
_LOW_MASK = np.uint64((1 << 45) - 1)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even (returned as fp64).

    Works on the fp64 bit pattern directly (no detour through fp32, so no double
    rounding): add half an ulp minus one plus the kept LSB, then clear the dropped bits.
    A carry out of the fraction correctly bumps the exponent."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise FloatingPointError("non-finite value reached a bf16 rounding point")
    tiny = (x != 0) & (np.abs(x) < 2.0 ** -126)
    if np.any(tiny):
        raise FloatingPointError("value below the bf16 normal range reached a rounding point")
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(_EXP_BITS_DROPPED)) & np.uint64(1)
    out = ((bits + _HALF_MINUS_ONE + lsb) & ~_LOW_MASK).view(np.float64)
    return out


def round_f32(x) -> np.ndarray:
    """Round fp64 values to the nearest fp32 value (numpy's IEEE cast, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def decode_bf16_bits(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------------------

@dataclass
class Layer:
    """One decoder layer plus LM head, weights held as fp64 (exact copies of the stored values)."""
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    precision: str            # "bf16" or "f32": the storage format of weights, cache and activations
    rope_base: float
    eps: float
    embed: np.ndarray         # [vocab, hidden]
    wq: np.ndarray            # [Hq*d, hidden]
    wk: np.ndarray            # [Hkv*d, hidden]
    wv: np.ndarray            # [Hkv*d, hidden]
    wo: np.ndarray            # [hidden, Hq*d]
    wg: np.ndarray            # [ffn, hidden]
    wu: np.ndarray            # [ffn, hidden]
    wd: np.ndarray            # [hidden, ffn]
    wlm: np.ndarray           # [vocab, hidden]

    def rnd(self, x):
        return round_bf16(x) if self.precision == "bf16" else round_f32(x)


def make_layer(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, weights: dict,
               precision="bf16", rope_base=10000.0, eps=1e-6, only=None) -> Layer:
    """Build a Layer from stored tensors (uint16 bf16 bits or float32 arrays).

    `weights` uses the library's packed layout: w_qkv rows are the Q heads, then the K
    heads, then the V heads; w_gate_up rows are gate then up.  `only` may name a subset
    of tensors to decode (the others are left as None)."""
    def dec(name):
        if only is not None and name not in only:
            return None
        w = weights[name]
        return decode_bf16_bits(w) if w.dtype == np.uint16 else np.asarray(w, dtype=np.float64)

    assert n_q_heads % n_kv_heads == 0
    qd, kd = n_q_heads * head_dim, n_kv_heads * head_dim
    wqkv = dec("w_qkv")
    wgu = dec("w_gate_up")
    return Layer(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, precision, rope_base, eps,
                 embed=dec("embed"),
                 wq=None if wqkv is None else wqkv[:qd],
                 wk=None if wqkv is None else wqkv[qd:qd + kd],
                 wv=None if wqkv is None else wqkv[qd + kd:qd + 2 * kd],
                 wo=dec("w_o"),
                 wg=None if wgu is None else wgu[:ffn],
                 wu=None if wgu is None else wgu[ffn:],
                 wd=dec("w_down"),
                 wlm=dec("w_lm"))


class Cache:
    """KV cache of one sequence: K, V as [Hkv, cap, d] fp64 holding stored values."""

    def __init__(self, n_kv_heads: int, cap: int, head_dim: int):
        self.K = np.zeros((n_kv_heads, cap, head_dim))
        self.V = np.zeros((n_kv_heads, cap, head_dim))
        self.length = 0
        self.cap = cap

    def copy(self) -> "Cache":
        c = Cache(self.K.shape[0], self.cap, self.K.shape[2])
        c.K[:] = self.K
        c.V[:] = self.V
        c.length = self.length
        return c


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis (gain fixed at 1)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_cos_sin(positions, head_dim: int, base: float):
    """cos/sin of the rotary angles p * base^(-2i/d), i < d/2, in fp64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Half-split rotary embedding of x [n, H, d] at absolute positions [n].

    Element i pairs with element i + d/2: (a, b) -> (a cos - b sin, b cos + a sin)."""
    d = x.shape[-1]
    c, s = rope_cos_sin(positions, d, base)
    c, s = c[:, None, :], s[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def qkv_rows(L: Layer, u: np.ndarray, positions):
    """Project normed rows u [n, hidden] and rotate: returns stored q [n,Hq,d], k, v [n,Hkv,d]."""
    n, d = u.shape[0], L.head_dim
    q = (u @ L.wq.T).reshape(n, L.n_q_heads, d)
    k = (u @ L.wk.T).reshape(n, L.n_kv_heads, d)
    v = (u @ L.wv.T).reshape(n, L.n_kv_heads, d)
    q = L.rnd(apply_rope(q, positions, L.rope_base))          # R2
    k = L.rnd(apply_rope(k, positions, L.rope_base))          # R3
    v = L.rnd(v)                                              # R3
    return q, k, v


def embed_norm(L: Layer, tokens):
    x = L.embed[np.asarray(tokens, dtype=np.int64)]
    return x, L.rnd(rms_norm(x, L.eps))                       # R1


def kv_group(L: Layer, h: int) -> int:
    """KV head that query head h reads: consecutive blocks of Hq/Hkv query heads share one."""
    return h // (L.n_q_heads // L.n_kv_heads)


def layer_block(L: Layer, x: np.ndarray, o: np.ndarray) -> dict:
    """Everything of a layer after attention: O projection + residual, SwiGLU MLP + residual,
    and the RMSNorm of the result (the next layer's normed input, or the final norm).
    x: layer input rows [n, hidden]; o: stored attention output."""
    h1 = round_f32(x + o @ L.wo.T)
    u2 = L.rnd(rms_norm(h1, L.eps))                           # R5
    act = L.rnd(silu(u2 @ L.wg.T) * (u2 @ L.wu.T))            # R6
    h2 = round_f32(h1 + act @ L.wd.T)
    hidden_out = L.rnd(h2)                                    # R7
    u3 = L.rnd(rms_norm(h2, L.eps))                           # R8
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": hidden_out, "u3": u3}


def lm_head(L: Layer, u3: np.ndarray) -> dict:
    """Logits of the final normed rows, their argmax (ties to the lowest id) and top-2 gap."""
    logits = round_f32(u3 @ L.wlm.T)
    return {"logits": logits, "argmax": argmax_lowest(logits), "top2_gap": top2_gap(logits)}


def tail(L: Layer, x: np.ndarray, o: np.ndarray) -> dict:
    """Everything after attention of a one-layer model: the layer block, then the LM head."""
    out = layer_block(L, x, o)
    out.update(lm_head(L, out["u3"]))
    return out


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Row argmax; among equal maxima the lowest index (numpy's argmax returns the first)."""
    return np.argmax(logits, axis=-1).astype(np.int64)


def top2_gap(logits: np.ndarray) -> np.ndarray:
    """Largest minus second-largest logit per row."""
    part = np.partition(logits, -2, axis=-1)
    return part[..., -1] - part[..., -2]


def masked_argmax(logits: np.ndarray, allowed: np.ndarray, vocab: int):
    """Argmax restricted to an allowed id set per row (Copy-as-Decode §2.3: at decision points
    the FSM intersects the model's logits with the tokens its state allows).  allowed [rows, A]
    holds ids; entries outside [0, vocab) are padding.  Ties go to the lowest id.  Returns the
    chosen id per row (-1 when a row allows nothing), the logits at the allowed slots (-inf for
    padding) and the gap between the best and second-best distinct allowed ids."""
    logits = np.asarray(logits, dtype=np.float64)
    allowed = np.asarray(allowed)
    rows, A = allowed.shape
    best = np.full(rows, -1, dtype=np.int64)
    vals = np.full((rows, A), -np.inf)
    gap = np.full(rows, np.inf)
    for r in range(rows):
        ids = sorted({int(a) for a in allowed[r] if 0 <= a < vocab})
        for k in range(A):
            a = int(allowed[r, k])
            if 0 <= a < vocab:
                vals[r, k] = logits[r, a]
        if ids:
            sub = logits[r, ids]
            best[r] = ids[int(np.argmax(sub))]                # first maximum = lowest id (ids sorted)
            if len(ids) > 1:
                srt = np.sort(sub)
                gap[r] = srt[-1] - srt[-2]
    return best, vals, gap


def softmax_checked(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (entries at -inf get weight 0); rows must sum to 1."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    p = e / np.sum(e, axis=-1, keepdims=True)
    if np.any(np.abs(np.sum(p, axis=-1) - 1.0) > 1e-12):
        raise AssertionError("softmax row does not sum to 1")
    return p


# ---------------------------------------------------------------------------------------
# caches built from a prefix
# ---------------------------------------------------------------------------------------

def cache_from_hidden(L: Layer, hidden: np.ndarray, cap: int) -> Cache:
    """Cache rows 0..n-1 from given hidden states: normed (R1), projected, rotated, stored."""
    c = Cache(L.n_kv_heads, cap, L.head_dim)
    u = L.rnd(rms_norm(np.asarray(hidden, dtype=np.float64), L.eps))
    pos = np.arange(u.shape[0])
    _, k, v = qkv_rows_kv_only(L, u, pos)
    c.K[:, : u.shape[0]] = k.transpose(1, 0, 2)
    c.V[:, : u.shape[0]] = v.transpose(1, 0, 2)
    c.length = u.shape[0]
    return c


def qkv_rows_kv_only(L: Layer, u: np.ndarray, positions):
    n, d = u.shape[0], L.head_dim
    k = (u @ L.wk.T).reshape(n, L.n_kv_heads, d)
    v = (u @ L.wv.T).reshape(n, L.n_kv_heads, d)
    return None, L.rnd(apply_rope(k, positions, L.rope_base)), L.rnd(v)


def cache_from_tokens(L: Layer, tokens, cap: int, chunk: int = 4096) -> Cache:
    """Cache rows for a token prefix at positions 0..n-1 (the K/V part of a prefill).

    With a single layer the cached K/V of a token depend only on its embedding and its
    position, so only the embedding, norm, K/V projections and RoPE are needed."""
    tokens = np.asarray(tokens)
    c = Cache(L.n_kv_heads, cap, L.head_dim)
    for s in range(0, len(tokens), chunk):
        t = tokens[s:s + chunk]
        _, u = embed_norm(L, t)
        _, k, v = qkv_rows_kv_only(L, u, np.arange(s, s + len(t)))
        c.K[:, s:s + len(t)] = k.transpose(1, 0, 2)
        c.V[:, s:s + len(t)] = v.transpose(1, 0, 2)
    c.length = len(tokens)
    return c


# ---------------------------------------------------------------------------------------
# forwards
# ---------------------------------------------------------------------------------------

def _decode_attend(L: Layer, cache: Cache, u: np.ndarray, p: int):
    """Decode-step attention of one normed row at position p: its K/V are written to slot p,
    then each query head attends to slots [0, p].  Returns q, k, v and the stored output."""
    q, k, v = qkv_rows(L, u, [p])
    cache.K[:, p] = k[0]
    cache.V[:, p] = v[0]
    o = np.zeros((L.n_q_heads, L.head_dim))
    for h in range(L.n_q_heads):
        g = kv_group(L, h)
        keys, vals = cache.K[g, : p + 1], cache.V[g, : p + 1]
        scores = keys @ q[0, h] / math.sqrt(L.head_dim)
        o[h] = softmax_checked(scores) @ vals
    return q, k, v, L.rnd(o.reshape(1, -1))                  # R4


def decode_one(L: Layer, cache: Cache, token: int) -> dict:
    """One autoregressive step: the token at position len is appended, then attends to
    slots [0, len] one query head at a time; len grows by one."""
    p = cache.length
    if p + 1 > cache.cap:
        raise ValueError("cache capacity exceeded")
    x, u = embed_norm(L, [token])
    q, k, v, o = _decode_attend(L, cache, u, p)
    cache.length = p + 1
    out = tail(L, x, o)
    out.update(q=q, k=k, v=v, o=o, u=u, x=x)
    return out


def span_layout(length: int, n: int, mode: str, W: int = 1, D: int = 0):
    """Slots, positions and the explicit [n, length + n] attention mask of a span forward.

    causal : row j sits at slot/position length + j and sees slots [0, length + j].
    block  : row (w, j) sits at slot length + w*D + j with position length + j; it sees the
             cached prefix [0, length) and slots length + w*D + j' for j' <= j."""
    S = length + n
    mask = np.zeros((n, S), dtype=bool)
    mask[:, :length] = True
    if mode == "causal":
        slots = length + np.arange(n)
        pos = slots.copy()
        for j in range(n):
            mask[j, length: length + j + 1] = True
    elif mode == "block":
        if W * D != n:
            raise ValueError("block mode needs n == W*D")
        slots = length + np.arange(n)
        pos = length + np.tile(np.arange(D), W)
        for w in range(W):
            for j in range(D):
                r = w * D + j
                mask[r, length + w * D: length + w * D + j + 1] = True
    else:
        raise ValueError(mode)
    return slots, pos, mask


def span_forward(L: Layer, cache: Cache, tokens, mode: str = "causal", W: int = 1, D: int = 0,
                 commit: bool = True) -> dict:
    """One parallel forward over n tokens (Copy-as-Decode §2.4; SwitchSD block verify).

    All n rows write K/V first (append-then-attend), then every row attends through the
    explicit mask of `span_layout`.  commit=True advances len by n (a copy span commits
    all of its tokens, acceptance being 1 by construction)."""
    tokens = np.asarray(tokens)
    n, base = len(tokens), cache.length
    if base + n > cache.cap:
        raise ValueError("cache capacity exceeded")
    slots, pos, mask = span_layout(base, n, mode, W, D)
    x, u = embed_norm(L, tokens)
    q, k, v, o = _span_attend(L, cache, u, pos, slots, mask)
    if commit:
        cache.length = base + n
    out = tail(L, x, o)
    out.update(q=q, k=k, v=v, o=o, u=u, x=x, positions=pos, slots=slots)
    return out


def _span_attend(L: Layer, cache: Cache, u: np.ndarray, pos, slots, mask):
    """Span attention of normed rows u: all rows write K/V to their slots first, then every
    row attends through the explicit mask.  Returns q, k, v and the stored output."""
    n = u.shape[0]
    q, k, v = qkv_rows(L, u, pos)
    cache.K[:, slots] = k.transpose(1, 0, 2)
    cache.V[:, slots] = v.transpose(1, 0, 2)
    S = mask.shape[1]
    o = np.zeros((n, L.n_q_heads, L.head_dim))
    for h in range(L.n_q_heads):
        g = kv_group(L, h)
        scores = q[:, h, :] @ cache.K[g, :S].T / math.sqrt(L.head_dim)
        scores = np.where(mask, scores, -np.inf)
        o[:, h, :] = softmax_checked(scores) @ cache.V[g, :S]
    return q, k, v, L.rnd(o.reshape(n, -1))                   # R4


# ---------------------------------------------------------------------------------------
# full-depth stacks: the same layer repeated with its own weights and cache
# ---------------------------------------------------------------------------------------
# Copy-as-Decode §2.4 and Table 11 run the span forward through whole models.  A stack is
# a list of layers: the embedding of the first and the LM head of the last are used.  Layer
# l > 0 takes the previous layer's residual output h2 as its input x and that output's RMSNorm
# u3 as its normed input (every norm has gain 1, so the next layer's input norm and the
# final norm are the same operation).  All caches of a stack hold the same length.

def stack_span_forward(layers: list, caches: list, tokens, mode: str = "causal", W: int = 1,
                       D: int = 0, commit: bool = True) -> dict:
    """One parallel forward of n tokens through every layer of a stack (causal span or
    block-triangular mask, as `span_forward`); commit=True advances every cache by n."""
    tokens = np.asarray(tokens)
    n, base = len(tokens), caches[0].length
    if any(c.length != base for c in caches):
        raise ValueError("stack caches disagree in length")
    if base + n > caches[0].cap:
        raise ValueError("cache capacity exceeded")
    slots, pos, mask = span_layout(base, n, mode, W, D)
    x, u = embed_norm(layers[0], tokens)
    for L, c in zip(layers, caches):
        _, _, _, o = _span_attend(L, c, u, pos, slots, mask)
        blk = layer_block(L, x, o)
        x, u = blk["h2"], blk["u3"]
    if commit:
        for c in caches:
            c.length = base + n
    blk.update(lm_head(layers[-1], u))
    blk.update(positions=pos, slots=slots)
    return blk


def stack_decode_one(layers: list, caches: list, token: int) -> dict:
    """One autoregressive step through a stack (decode-step attention in every layer)."""
    p = caches[0].length
    if any(c.length != p for c in caches):
        raise ValueError("stack caches disagree in length")
    if p + 1 > caches[0].cap:
        raise ValueError("cache capacity exceeded")
    x, u = embed_norm(layers[0], [token])
    for L, c in zip(layers, caches):
        _, _, _, o = _decode_attend(L, c, u, p)
        blk = layer_block(L, x, o)
        x, u = blk["h2"], blk["u3"]
    for c in caches:
        c.length = p + 1
    blk.update(lm_head(layers[-1], u))
    return blk


def stack_prefill(layers: list, tokens, cap: int, chunk: int = 512) -> list:
    """Caches of every layer for a token prefix: causal span forwards over chunks of it."""
    caches = [Cache(L.n_kv_heads, cap, L.head_dim) for L in layers]
    tokens = np.asarray(tokens)
    for s in range(0, len(tokens), chunk):
        stack_span_forward(layers, caches, tokens[s:s + chunk], "causal")
    return caches


# ---------------------------------------------------------------------------------------
# n-gram draft lookup (PLD page, "The n-gram match, precisely"; SwitchSD kappa-gram gate)
# ---------------------------------------------------------------------------------------

def ngram_lookup(ctx, length: int, n: int, W: int, D: int):
    """Most-recent-first suffix match.

    The suffix is ctx[length-n:length].  Candidate starts run j = length-n-1 down to 0
    (so at least one continuation token exists and the suffix does not match itself);
    the first W hits are kept.  Draft w is ctx[j+n : min(j+n+D, length)], padded with 0.
    Returns drafts [W, D], draft_len [W], match_pos [W] (-1 where there is no hit)."""
    ctx = np.asarray(ctx)
    drafts = np.zeros((W, D), dtype=np.int64)
    dlen = np.zeros(W, dtype=np.int64)
    mpos = np.full(W, -1, dtype=np.int64)
    if length < n + 1:
        return drafts, dlen, mpos
    suffix = ctx[length - n: length]
    found = 0
    for j in range(length - n - 1, -1, -1):
        if found == W:
            break
        if np.array_equal(ctx[j: j + n], suffix):
            m = min(D, length - (j + n))
            drafts[found, :m] = ctx[j + n: j + n + m]
            dlen[found] = m
            mpos[found] = j
            found += 1
    return drafts, dlen, mpos


def ngram_lookup_longest(ctx, length: int, n_max: int, n_min: int, W: int, D: int):
    """Longest-match policy (PLD page, "The n-gram match, precisely": with several matches a
    common policy prefers the most recent or the longest; n is often 1-3).  Reading: try the
    suffix lengths n = n_max, n_max-1, ..., n_min in turn and keep the most-recent-first hits of
    the first length that has any.  Returns drafts, draft_len, match_pos as `ngram_lookup`, and
    the suffix length used (0 when no length matches)."""
    for n in range(n_max, n_min - 1, -1):
        d, l, m = ngram_lookup(ctx, length, n, W, D)
        if m[0] >= 0:
            return d, l, m, n
    d, l, m = ngram_lookup(ctx, length, n_min, W, D)
    return d, l, m, 0


def ngram_lookup_bruteforce(ctx, length: int, n: int, W: int, D: int):
    """Second, independently written lookup used to pin `ngram_lookup` on tiny inputs:
    list every (start, continuation) pair whose n tokens equal the suffix, newest first."""
    seq = [int(t) for t in np.asarray(ctx)[:length]]
    hits = []
    if length >= n + 1:
        suf = tuple(seq[length - n:])
        for j in range(0, length - n):
            if tuple(seq[j:j + n]) == suf:
                hits.append((j, seq[j + n: j + n + D]))
    hits.sort(key=lambda t: -t[0])
    hits = hits[:W]
    drafts = [c + [0] * (D - len(c)) for _, c in hits] + [[0] * D] * (W - len(hits))
    dlen = [len(c) for _, c in hits] + [0] * (W - len(hits))
    mpos = [j for j, _ in hits] + [-1] * (W - len(hits))
    return np.array(drafts, dtype=np.int64).reshape(W, D), np.array(dlen, dtype=np.int64), \
        np.array(mpos, dtype=np.int64)


# ---------------------------------------------------------------------------------------
# acceptance (PLD page, "Verification in a single parallel pass"; SwitchSD longest prefix)
# ---------------------------------------------------------------------------------------

def accept_causal(draft, draft_len: int, pred):
    """Forward tokens were [g, d_1..d_k]; pred[i] is the target's argmax at forward index i.
    a counts the leading drafts that agree (d_{a+1} == pred[a]); emit d_1..d_a then pred[a].
    Returns (a, emitted list of a+1 tokens)."""
    a = 0
    while a < draft_len and int(draft[a]) == int(pred[a]):
        a += 1
    return a, [int(t) for t in draft[:a]] + [int(pred[a])]


def accept_block(drafts, draft_lens, pred, first_pred: int, D: int):
    """Block-triangular verify: candidate w occupies forward rows w*D..w*D+D-1; its first
    token is checked against first_pred (the target's prediction at the cached anchor) and
    token j > 0 against pred[w*D + j - 1].  The longest run wins, ties to the lowest w.
    Returns (a_star, w_star, emitted list of a_star+1 tokens, per-candidate a)."""
    W = len(draft_lens)
    a_all = []
    for w in range(W):
        a = 0
        while a < int(draft_lens[w]):
            want = first_pred if a == 0 else int(pred[w * D + a - 1])
            if int(drafts[w][a]) != want:
                break
            a += 1
        a_all.append(a)
    w_star = int(np.argmax(a_all))               # first maximum
    a_star = a_all[w_star]
    bonus = first_pred if a_star == 0 else int(pred[w_star * D + a_star - 1])
    emitted = [int(t) for t in drafts[w_star][:a_star]] + [bonus]
    return a_star, w_star, emitted, a_all


def commit_block(cache: Cache, w_star: int, a_star: int, D: int):
    """Move the winner's accepted rows from slot len + w*D + j to len + j (j < a*); len += a*.
    Their RoPE position is already len + j, so the move is a plain copy."""
    base = cache.length
    src = base + w_star * D + np.arange(a_star)
    dst = base + np.arange(a_star)
    cache.K[:, dst] = cache.K[:, src]
    cache.V[:, dst] = cache.V[:, src]
    cache.length = base + a_star


def pld_speedup(f: float, L: float) -> float:
    """Copy-rate speedup of the PLD page: 1 / (f/L + (1 - f))."""
    return 1.0 / (f / L + (1.0 - f))


# ---------------------------------------------------------------------------------------
# stochastic verification (PLD page, "Speculative decoding in one breath": with the proper
# rejection-sampling correction the accepted text keeps the target's sampling distribution)
# ---------------------------------------------------------------------------------------
# The drafter is deterministic (a retrieved continuation), so its proposal distribution q is
# one-hot on the draft token d.  The standard correction then reads: accept d with probability
# min(1, p(d) / q(d)) = p(d); on rejection draw from the residual max(0, p - q), renormalised,
# which is p with d removed; after an accepted draft draw the bonus token from p.  Here p is
# softmax(logits / temperature) of the row.  Draws use the Gumbel-max form (the argmax of
# logits / T plus independent Gumbel noise is a sample of p; restricted to x != d it is a sample
# of the residual) with uniforms from the Philox4x32-10 counter-based generator.

_PHILOX_M0, _PHILOX_M1 = 0xD2511F53, 0xCD9E8D57      # round multipliers (Salmon et al., SC'11)
_PHILOX_W0, _PHILOX_W1 = 0x9E3779B9, 0xBB67AE85      # key increments (golden ratio, sqrt(3) - 1)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
    easy as 1, 2, 3", SC'11).  ctr: uint32 array [..., 4]; key: uint32 pair.  Each round
    multiplies words 0 and 2 by the round multipliers into 64-bit products and mixes:
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key is bumped by the
    Weyl increments between rounds.  Returns uint32 [..., 4]."""
    c = np.asarray(ctr, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        p0 = np.uint64(_PHILOX_M0) * c0
        p1 = np.uint64(_PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if r < 9:
            k0 = (k0 + np.uint64(_PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(_PHILOX_W1)) & mask
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniform_from_bits(bits):
    """(0, 1) uniform from 32 random bits: the top 23 bits k give (2k + 1) / 2^24, exactly
    representable in fp32 and never 0 or 1."""
    k = (np.asarray(bits, dtype=np.uint64) >> np.uint64(9)).astype(np.float64)
    return (2.0 * k + 1.0) / 16777216.0


def sample_uniforms(seed: int, b: int, pos, ids, purpose: int):
    """Uniforms of draw (sequence b, absolute position pos, vocabulary id, purpose): Philox
    counter (id // 4, pos, b, purpose), key (seed low word, seed high word), output word id % 4.
    purpose 0 = Gumbel noise of a logit, 1 = the acceptance test of a row (id 0)."""
    ids = np.asarray(ids, dtype=np.int64)
    pos = np.broadcast_to(np.asarray(pos, dtype=np.int64), ids.shape)
    ctr = np.stack([ids // 4, pos, np.full(ids.shape, b), np.full(ids.shape, purpose)], axis=-1)
    out = philox4x32_10(ctr.astype(np.uint64), (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    word = np.take_along_axis(out, (ids % 4)[..., None], axis=-1)[..., 0]
    return uniform_from_bits(word)


def sampled_predictions(logits, tokens, draft_len: int, temperature: float, seed: int, b: int, base: int):
    """The per-row tokens a stochastic verifier compares and emits, for one sequence's forward
    rows over tokens [g, d_1..d_k] at absolute positions base + i.

    Row i < draft_len holds the draft d = tokens[i + 1]: it keeps d with probability p_i(d) (the
    acceptance test u < p_i(d)), else it is a draw from p_i without d.  Row i >= draft_len is a
    plain draw from p_i.  With these predictions the greedy left-to-right scan
    (`accept_causal`) emits exactly the stochastic result: it continues while a row kept its
    draft and emits the first replacement, or the bonus draw after the last draft.
    Returns (pred, y, z, p_draft, u): y = plain draws, z = draws without the draft."""
    logits = np.asarray(logits, dtype=np.float64)
    n, V = logits.shape
    s = logits / temperature
    ids = np.arange(V)
    pred = np.zeros(n, dtype=np.int64)
    y = np.zeros(n, dtype=np.int64)
    z = np.full(n, -1, dtype=np.int64)
    pd = np.full(n, np.nan)
    u = np.full(n, np.nan)
    for i in range(n):
        g = -np.log(-np.log(sample_uniforms(seed, b, base + i, ids, 0)))
        pert = s[i] + g
        y[i] = int(np.argmax(pert))
        if i < draft_len:
            d = int(tokens[i + 1])
            m = np.max(s[i])
            lse = m + np.log(np.sum(np.exp(s[i] - m)))
            pd[i] = math.exp(s[i, d] - lse)
            u[i] = float(sample_uniforms(seed, b, base + i, [0], 1)[0])
            alt = pert.copy()
            alt[d] = -np.inf
            z[i] = int(np.argmax(alt))
            pred[i] = d if u[i] < pd[i] else z[i]
        else:
            pred[i] = y[i]
    return pred, y, z, pd, u


def sampled_margins(logits, tokens, draft_len: int, temperature: float, seed: int, b: int, base: int):
    """How firmly `sampled_predictions` decides each row: the gap between the best and the
    second-best Gumbel-perturbed tempered logit over all ids (y_gap) and over the ids other than
    the draft (z_gap, drafted rows only), and |u - p(d)| / p(d) of the acceptance test."""
    logits = np.asarray(logits, dtype=np.float64)
    n, V = logits.shape
    s = logits / temperature
    ids = np.arange(V)
    y_gap = np.zeros(n)
    z_gap = np.full(n, np.inf)
    acc_margin = np.full(n, np.inf)
    _, _, _, pd, u = sampled_predictions(logits, tokens, draft_len, temperature, seed, b, base)
    for i in range(n):
        pert = s[i] - np.log(-np.log(sample_uniforms(seed, b, base + i, ids, 0)))
        top = np.sort(pert)[-2:]
        y_gap[i] = top[1] - top[0]
        if i < draft_len:
            alt = pert.copy()
            alt[int(tokens[i + 1])] = -np.inf
            top = np.sort(alt)[-2:]
            z_gap[i] = top[1] - top[0]
            acc_margin[i] = abs(u[i] - pd[i]) / pd[i]
    return y_gap, z_gap, acc_margin
