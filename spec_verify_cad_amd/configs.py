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
