"""Seeded synthetic inputs for the span-commit / verify path.

This module only draws random data: weights, token streams, contexts with planted
repeats, span-length schedules and random hidden states.  It holds none of the
method's arithmetic (no normalisation, projection, position encoding, attention,
lookup or acceptance), so both the CPU oracle and the HIP path can be fed from it
without sharing any of the computation.

Every generator is a pure function of its seed.  Large tensors are drawn in
fixed-size row blocks, each from its own generator keyed by (seed, tensor id,
block), so a block of rows can be regenerated alone.

Data conventions:
  * weights and embeddings ~ N(0, 0.02^2), drawn in fp32 and rounded once to
    bf16 (round-to-nearest-even, via torch's CPU conversion) for bf16 layers;
    both paths then read the same bits;
  * bf16 tensors are returned as numpy uint16 bit patterns;
  * fp32 tensors (the tiny fp32 layer) are returned as numpy float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ROW_BLOCK = 4096  # rows per independently seeded block

# tensor ids used in the generator keys
_TID = {"embed": 1, "w_qkv": 2, "w_o": 3, "w_gate_up": 4, "w_down": 5, "w_lm": 6,
        "hidden": 7, "tokens": 8, "context": 9, "program": 10}


def _rng(seed: int, tid: str, block: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TID[tid], int(block)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), rounded by torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_matrix(seed: int, tid: str, rows: int, cols: int, std: float = 0.02,
                  dtype: str = "bf16", row_lo: int = 0, row_hi: int | None = None) -> np.ndarray:
    """Rows [row_lo, row_hi) of a [rows, cols] N(0, std^2) matrix.

    Returns uint16 bf16 bits (dtype="bf16") or float32 (dtype="f32")."""
    row_hi = rows if row_hi is None else row_hi
    assert 0 <= row_lo <= row_hi <= rows
    out = np.empty((row_hi - row_lo, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    b0, b1 = row_lo // ROW_BLOCK, (row_hi + ROW_BLOCK - 1) // ROW_BLOCK
    for blk in range(b0, b1):
        r0 = blk * ROW_BLOCK
        nr = min(ROW_BLOCK, rows - r0)
        vals = _rng(seed, tid, blk).standard_normal((nr, cols), dtype=np.float32) * np.float32(std)
        lo, hi = max(row_lo, r0), min(row_hi, r0 + nr)
        part = vals[lo - r0:hi - r0]
        out[lo - row_lo:hi - row_lo] = f32_to_bf16_bits(part) if dtype == "bf16" else part
    return out


@dataclass(frozen=True)
class LayerShape:
    """Shape of one pre-norm decoder layer plus its LM head."""
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str = "bf16"          # "bf16" or "f32"
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def elt_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def layer_params(self) -> int:
        h, d = self.hidden, self.head_dim
        return (self.qkv_out * h + h * self.n_q_heads * d + 2 * self.ffn * h + h * self.ffn)

    def lm_params(self) -> int:
        return self.vocab * self.hidden


def weight_shapes(s: LayerShape) -> dict:
    """Row-major [out, in] shapes of every tensor the layer reads."""
    return {
        "embed": (s.vocab, s.hidden),
        "w_qkv": (s.qkv_out, s.hidden),                    # rows: Q heads, then K heads, then V heads
        "w_o": (s.hidden, s.n_q_heads * s.head_dim),
        "w_gate_up": (2 * s.ffn, s.hidden),                 # rows: gate, then up
        "w_down": (s.hidden, s.ffn),
        "w_lm": (s.vocab, s.hidden),
    }


def layer_weights(s: LayerShape, seed: int, names=None) -> dict:
    """All weights of a layer, N(0, 0.02^2), seeded."""
    shapes = weight_shapes(s)
    names = list(shapes) if names is None else names
    return {n: normal_matrix(seed, n, *shapes[n], dtype=s.dtype) for n in names}


def hidden_states(seed: int, count: int, width: int) -> np.ndarray:
    """Random hidden states ~ N(0, 1), fp32 [count, width] (source of a synthetic cache)."""
    return _rng(seed, "hidden").standard_normal((count, width), dtype=np.float32)


def uniform_tokens(seed: int, count: int, vocab: int, stream: int = 0) -> np.ndarray:
    return _rng(seed, "tokens", stream).integers(0, vocab, size=count, dtype=np.int64).astype(np.int32)


def zipf_ranks(rng: np.random.Generator, count: int, vocab: int, s: float) -> np.ndarray:
    """Bounded Zipf(s) over ranks 1..vocab by inverse-CDF sampling; returns 0-based ranks."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    r = np.searchsorted(cdf, rng.random(count), side="right")
    return np.minimum(r, vocab - 1)


def planted_context(seed: int, length: int, vocab: int, frac: float, min_copy: int, max_copy: int,
                    background: str = "uniform", zipf_s: float = 1.1, stream: int = 0) -> tuple:
    """int32 context with verbatim repeats planted from strictly earlier positions.

    Background tokens are uniform over the vocabulary or a bounded Zipf mapped to ids
    through a seeded permutation.  Copies of length U{min_copy..max_copy} are planted at
    random destinations, each taken from a random earlier source, until at least `frac`
    of the positions lie inside a copy.  Returns (ctx, covered_mask)."""
    rng = _rng(seed, "context", stream)
    if background == "uniform":
        ctx = rng.integers(0, vocab, size=length, dtype=np.int64)
    elif background == "zipf":
        perm = rng.permutation(vocab)
        ctx = perm[zipf_ranks(rng, length, vocab, zipf_s)]
    else:
        raise ValueError(background)
    ctx = ctx.astype(np.int32)
    covered = np.zeros(length, dtype=bool)
    target = int(math.ceil(frac * length))
    guard = 0
    while covered.sum() < target and guard < 100000:
        guard += 1
        n = int(rng.integers(min_copy, max_copy + 1))
        if 2 * n + 1 > length:
            continue
        dst = int(rng.integers(n, length - n + 1))
        src = int(rng.integers(0, dst - n + 1))      # source ends at or before dst
        ctx[dst:dst + n] = ctx[src:src + n]
        covered[dst:dst + n] = True
    return ctx, covered


def plant_anchor_repeats(ctx: np.ndarray, seed: int, kappa: int, copies: int, min_len: int,
                         max_len: int, stream: int = 0) -> np.ndarray:
    """Make the final `kappa` tokens of `ctx` recur at least `copies` times earlier.

    Each planted occurrence copies the anchor kappa-gram followed by a fresh random
    continuation of length U{min_len..max_len} drawn from the context itself, so the
    candidates that follow the occurrences differ from one another."""
    rng = _rng(seed, "context", 1000 + stream)
    ctx = ctx.copy()
    L = len(ctx)
    anchor = ctx[L - kappa:].copy()
    span = L - kappa - max_len - kappa - 1
    starts = np.sort(rng.choice(np.arange(0, span, kappa + max_len + 1), size=copies, replace=False))
    for st in starts:
        ctx[st:st + kappa] = anchor
        n = int(rng.integers(min_len, max_len + 1))
        src = int(rng.integers(0, L - n))
        ctx[st + kappa:st + kappa + n] = ctx[src:src + n]
    ctx[L - kappa:] = anchor
    return ctx


def cad_program(seed: int, doc_len: int, total_out: int, median: float, sigma: float,
                max_span: int, gen_min: int, gen_max: int) -> list:
    """Seeded Copy-as-Decode op schedule: alternating ("copy", src, n) and ("gen", g) ops.

    Copy lengths are clip(round(exp(ln(median) + sigma*z)), 1, max_span) with z ~ N(0,1);
    copy sources are uniform in the document; gen lengths are U{gen_min..gen_max}.
    Ops alternate copy, gen, copy, ... and stop at `total_out` output tokens, the last
    op truncated to fit."""
    rng = _rng(seed, "program")
    ops, out = [], 0
    copy_turn = True
    while out < total_out:
        if copy_turn:
            n = int(np.clip(round(math.exp(math.log(median) + sigma * rng.standard_normal())), 1, max_span))
            n = min(n, total_out - out, doc_len)
            src = int(rng.integers(0, doc_len - n + 1))
            ops.append(("copy", src, n))
        else:
            g = int(rng.integers(gen_min, gen_max + 1))
            g = min(g, total_out - out)
            ops.append(("gen", g))
            n = g
        out += n
        copy_turn = not copy_turn
    return ops


# Structural literals of the Copy-as-Decode grammar as single token ids (Copy-as-Decode,
# Appendix A, "Qwen2.5 token identifiers").
CAD_TOK = {"LT": 27, "LT_SLASH": 522, "GT": 29, "COPY": 8560, "GEN": 4370, "PROGRAM": 14906,
           "SPACE_LINES": 5128, "EQ_QUOTE": 428, "QUOTE_SLASH": 9685, "SLASH_GT": 2577}


def _char_id(c: str) -> int:
    """Single printable characters in byte order, id = code - 33: the order that puts "<" at 27
    and ">" at 29 in the table above (digit, hyphen and quote ids are not on the page)."""
    return ord(c) - 33


CAD_DIGITS = tuple(_char_id(c) for c in "0123456789")
CAD_HYPHEN = _char_id("-")
CAD_QUOTE = _char_id('"')
LINE_TOKENS = 10   # document tokens per line, for the line numbers a copy tag carries


@dataclass(frozen=True)
class ProgramForward:
    """One forward of a Copy-as-Decode program.

    Its input is `lits` followed by the document tokens doc[src:src+n] when `doc` = (src, n),
    or, when `from_prev`, the single token the previous forward chose.  The decision after its
    last row is restricted to `allowed` (a masked step) or unrestricted (None)."""
    role: str
    lits: tuple = ()
    doc: tuple | None = None
    from_prev: bool = False
    allowed: tuple | None = None

    @property
    def n(self) -> int:
        return 1 if self.from_prev else len(self.lits) + (self.doc[1] if self.doc else 0)


def cad_program_forwards(ops: list, line_tokens: int = LINE_TOKENS) -> list:
    """The forwards a Copy-as-Decode program of `ops` runs after its prompt (Copy-as-Decode §2.3
    step types and Appendix A states), with every choice a trained model would make taken from
    the op schedule; only the <gen> bodies are the model's own tokens.

    Per op: feed "<" and decide the op type in {copy, gen}.  A copy then feeds the forced
    template (copy, " lines", '="') and decides the first digit; feeds each character of the
    line range "i-j" (i, j = 1-based lines of `line_tokens` tokens), deciding the next one
    (digits; digits or "-" inside the first number; digits or the closing quote inside the
    second); and finally feeds the closing quote, the forced "/>" and the copied tokens in one
    splice forward that decides the next op boundary in {"<", "</"}.  A gen feeds the forced
    (gen, ">"), then its g body tokens, each the previous forward's free choice, then the
    closing literal "</", gen, ">" one token at a time; the forward that feeds ">" decides the
    next boundary.  After the last op the forced terminator ("</", program, ">") closes it."""
    T = CAD_TOK
    boundary = (T["LT"], T["LT_SLASH"])
    digits = CAD_DIGITS
    out = []
    for op in ops:
        out.append(ProgramForward("op_type", (T["LT"],), allowed=(T["COPY"], T["GEN"])))
        if op[0] == "copy":
            _, src, n = op
            rng = f"{src // line_tokens + 1}-{(src + n - 1) // line_tokens + 1}"
            out.append(ProgramForward("copy_open", (T["COPY"], T["SPACE_LINES"], T["EQ_QUOTE"]), allowed=digits))
            second = False
            for ch in rng:
                if ch == "-":
                    second = True
                    nxt = digits
                else:
                    nxt = digits + ((CAD_QUOTE,) if second else (CAD_HYPHEN,))
                out.append(ProgramForward("line_char", (_char_id(ch),), allowed=nxt))
            out.append(ProgramForward("splice", (CAD_QUOTE, T["SLASH_GT"]), doc=(src, n), allowed=boundary))
        else:
            g = op[1]
            out.append(ProgramForward("gen_open", (T["GEN"], T["GT"])))
            out += [ProgramForward("gen_body", from_prev=True) for _ in range(g)]
            out.append(ProgramForward("gen_close", (T["LT_SLASH"],)))
            out.append(ProgramForward("gen_close", (T["GEN"],)))
            out.append(ProgramForward("gen_close", (T["GT"],), allowed=boundary))
    out.append(ProgramForward("close", (T["LT_SLASH"], T["PROGRAM"], T["GT"])))
    return out
