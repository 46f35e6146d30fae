"""The five synthetic workloads of the span-commit / verify path, as plain data.

Shapes follow the models the Copy-as-Decode page benchmarks (Qwen2.5-1.5B and -7B,
"Kernel microbenchmark" paragraph and Table 11): one decoder layer of that shape plus
its LM head.  Workload parameters (span lengths, n-gram order, draft length, number
of candidates) come from the Copy-as-Decode page (Table 2 span statistics), the PLD
page ("The n-gram match, precisely": n often 1-3, k about 10) and the SwitchSD page
(kappa = 5 structural gate, W recency-ranked candidates of length D).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .synth import LayerShape

TINY = LayerShape(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=1024, vocab=1024, dtype="f32")
QWEN15 = LayerShape(hidden=1536, n_q_heads=12, n_kv_heads=2, head_dim=128, ffn=8960, vocab=151936)
QWEN7 = LayerShape(hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064)
# small bf16 layer for parity at sizes the oracle finishes in seconds: several tiles
# in every dimension plus ragged tails (vocab and ffn are not multiples of the tiles)
SMALL = LayerShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1376, vocab=5003)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    seed: int
    cache_len: int
    spans: tuple = ()
    extra: dict = field(default_factory=dict)


CONFIGS = {
    # tiny fp32 layer: cache of 128 rows from random hidden states, one copy span of 8
    "tiny_f32": Workload("tiny_f32", TINY, 1001, 128, (8,), {"corrupt_pos": 5}),
    # 1.5B-shaped layer, L=2048 prefix, copy spans swept over N
    "qwen15_span": Workload("qwen15_span", QWEN15, 1002, 2048, (8, 16, 32, 64, 128, 256, 512)),
    # 7B-shaped layer, Copy-as-Decode program over a 4096-token document
    "qwen7_cad_program": Workload("qwen7_cad_program", QWEN7, 1003, 4096, (),
                                  {"doc_len": 4096, "total_out": 4096, "median": 24.0, "sigma": 0.855,
                                   "max_span": 512, "gen_min": 1, "gen_max": 8}),
    # 7B-shaped layer, block-triangular verify of W=4 candidates x D=8 at L=4096
    "qwen7_block_verify": Workload("qwen7_block_verify", QWEN7, 1004, 4096, (),
                                   {"ctx_len": 4096, "frac": 0.30, "min_copy": 5, "max_copy": 64,
                                    "kappa": 5, "W": 4, "D": 8}),
    # 1.5B-shaped layer, 64 sequences x 32768-token contexts, PLD n=3, k=10, 32 rounds
    "qwen15_pld_batch": Workload("qwen15_pld_batch", QWEN15, 1005, 32768, (),
                                 {"B": 64, "ctx_len": 32768, "frac": 0.40, "min_copy": 8, "max_copy": 256,
                                  "zipf_s": 1.1, "n": 3, "k": 10, "rounds": 32}),
}


# ---------------------------------------------------------------------------------------
# input recipes of the workloads (seeded data only; shared by the benchmark and the tests)
# ---------------------------------------------------------------------------------------

def copy_sweep_inputs(wl: Workload, spans=None, extra_tail: int = 4096):
    """Copy-span sweep: a uniform random document whose first cache_len tokens fill the
    cache, and for each span length N a span copied from a random later place of it.
    Returns (doc, prefix, [span tokens per N])."""
    import numpy as np
    from . import synth
    spans = wl.spans if spans is None else spans
    doc = synth.uniform_tokens(wl.seed, wl.cache_len + extra_tail, wl.shape.vocab, stream=3)
    rng = np.random.default_rng(wl.seed)
    srcs = [int(rng.integers(wl.cache_len, len(doc) - N)) for N in spans]
    return doc, doc[:wl.cache_len], [doc[s:s + N] for s, N in zip(srcs, spans)]


def block_verify_context(wl: Workload):
    """Context of the block-triangular verify: uniform background, planted verbatim repeats
    covering the configured fraction, and the final kappa-gram planted five more times with
    different continuations (so at least W candidates exist)."""
    from . import synth
    e = wl.extra
    ctx, _ = synth.planted_context(wl.seed, e["ctx_len"], wl.shape.vocab, e["frac"], e["min_copy"], e["max_copy"],
                                   "uniform")
    return synth.plant_anchor_repeats(ctx, wl.seed, e["kappa"], 5, e["D"], e["max_copy"])


def pld_contexts(wl: Workload, B=None):
    """Contexts of the batched PLD workload: per-sequence seed streams, bounded Zipf
    background, planted copies covering the configured fraction, and a final planted copy
    that runs to the end of the context, so every sequence starts mid-copy (the state prompt
    lookup targets: the suffix has an earlier occurrence).  Returns [B, ctx_len]."""
    import numpy as np
    from . import synth
    e = wl.extra
    B = e["B"] if B is None else B
    out = []
    for b in range(B):
        ctx, _ = synth.planted_context(wl.seed, e["ctx_len"], wl.shape.vocab, e["frac"], e["min_copy"],
                                       e["max_copy"], "zipf", e["zipf_s"], stream=b)
        rng = np.random.default_rng([wl.seed, 77, b])
        n = int(rng.integers(e["min_copy"], e["max_copy"] + 1))
        src = int(rng.integers(0, len(ctx) - 2 * n))
        ctx[len(ctx) - n:] = ctx[src:src + n]
        out.append(ctx)
    return np.stack(out)


def cad_program_inputs(wl: Workload):
    """Document and op schedule of the Copy-as-Decode program workload."""
    from . import synth
    e = wl.extra
    doc = synth.uniform_tokens(wl.seed, e["doc_len"], wl.shape.vocab, stream=5)
    ops = synth.cad_program(wl.seed, e["doc_len"], e["total_out"], e["median"], e["sigma"], e["max_span"],
                            e["gen_min"], e["gen_max"])
    return doc, ops
