"""Shared test fixtures: seeded layers and caches (inputs only; no method arithmetic)."""
import numpy as np

import oracle as O
from spec_verify_cad_amd import synth
from spec_verify_cad_amd.synth import LayerShape


def oracle_layer(shape: LayerShape, weights: dict, **kw) -> O.Layer:
    return O.make_layer(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                        shape.vocab, weights, precision=shape.dtype, rope_base=shape.rope_base,
                        eps=shape.rms_eps, **kw)


def small_layer(shape: LayerShape, seed: int):
    w = synth.layer_weights(shape, seed)
    return w, oracle_layer(shape, w)
