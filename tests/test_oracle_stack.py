"""Pins of the oracle's full-depth stack (Copy-as-Decode §2.4 and Table 11 run the span
forward through whole models).

* A one-layer stack is the one-layer model.
* Copy-as-Decode Appendix K at depth: a span forward of N tokens through the stack equals N
  decode steps through it, in every layer's cache and in the outputs.
* A layer whose O and down projections are zero passes its input through unchanged (both
  residual branches vanish), so a stack of one real layer and such layers reproduces the
  one-layer model, and their caches hold the K/V of the first layer's output rows.
* SwitchSD block verify at depth: each candidate's rows equal a causal forward of that
  candidate alone on the same prefix."""
import numpy as np
import pytest

import oracle as O
from spec_verify_cad_amd import synth
from spec_verify_cad_amd.synth import LayerShape

from helpers import oracle_layer

MINI = LayerShape(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=192, vocab=211)
MINI_F32 = LayerShape(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=192, vocab=211, dtype="f32")


def _stack(shape, seed, n):
    return [oracle_layer(shape, synth.layer_weights(shape, seed + l)) for l in range(n)]


def _caches(layers, cap):
    return [O.Cache(L.n_kv_heads, cap, L.head_dim) for L in layers]


def test_one_layer_stack_is_the_one_layer_model():
    (L,) = _stack(MINI, 3, 1)
    ctx = synth.uniform_tokens(3, 30, MINI.vocab)
    span = synth.uniform_tokens(3, 7, MINI.vocab, stream=1)
    c = O.cache_from_tokens(L, ctx, 64)
    (sc,) = O.stack_prefill([L], ctx, 64)
    np.testing.assert_array_equal(sc.K[:, :30], c.K[:, :30])
    a = O.span_forward(L, c, span)
    b = O.stack_span_forward([L], [sc], span)
    for k in ("hidden_out", "logits", "argmax"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    d = O.decode_one(L, c, int(span[0]))
    e = O.stack_decode_one([L], [sc], int(span[0]))
    np.testing.assert_array_equal(d["logits"], e["logits"])


@pytest.mark.parametrize("shape", [MINI, MINI_F32])
def test_stack_span_equals_sequential_decode(shape):
    layers = _stack(shape, 20, 3)
    ctx = synth.uniform_tokens(21, 25, shape.vocab)
    span = synth.uniform_tokens(21, 9, shape.vocab, stream=1)
    c1 = O.stack_prefill(layers, ctx, 48, chunk=10)           # chunked causal prefill
    c2 = [c.copy() for c in c1]
    s = O.stack_span_forward(layers, c1, span)
    steps = [O.stack_decode_one(layers, c2, int(t)) for t in span]
    tol = 1e-12 if shape.dtype == "f32" else 0.0
    for k in ("hidden_out", "logits"):
        np.testing.assert_allclose(s[k], np.concatenate([d[k] for d in steps]), rtol=0, atol=tol, err_msg=k)
    np.testing.assert_array_equal(s["argmax"], np.concatenate([d["argmax"] for d in steps]))
    for a, b in zip(c1, c2):
        assert a.length == b.length == 34
        np.testing.assert_allclose(a.K, b.K, rtol=0, atol=tol)
        np.testing.assert_allclose(a.V, b.V, rtol=0, atol=tol)


def test_prefill_chunking_does_not_change_the_caches():
    layers = _stack(MINI, 40, 2)
    ctx = synth.uniform_tokens(41, 37, MINI.vocab)
    a = O.stack_prefill(layers, ctx, 40, chunk=37)
    b = O.stack_prefill(layers, ctx, 40, chunk=8)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.K, y.K)
        np.testing.assert_array_equal(x.V, y.V)


def test_pass_through_layers_reproduce_the_one_layer_model():
    w0 = synth.layer_weights(MINI, 50)
    L0 = oracle_layer(MINI, w0)
    rest = []
    for l in range(1, 3):
        w = synth.layer_weights(MINI, 50 + l)
        w["w_o"] = np.zeros_like(w["w_o"])
        w["w_down"] = np.zeros_like(w["w_down"])
        w["w_lm"] = w0["w_lm"]
        rest.append(oracle_layer(MINI, w))
    layers = [L0] + rest
    ctx = synth.uniform_tokens(51, 20, MINI.vocab)
    span = synth.uniform_tokens(51, 6, MINI.vocab, stream=1)
    caches = O.stack_prefill(layers, ctx, 32)
    one = O.cache_from_tokens(L0, ctx, 32)
    pre = O.span_forward(L0, O.cache_from_tokens(L0, [], 32), ctx)          # layer 0 over the prefix
    s = O.stack_span_forward(layers, caches, span)
    r = O.span_forward(L0, one, span)
    for k in ("h2", "hidden_out", "logits", "argmax"):
        np.testing.assert_array_equal(s[k], r[k], err_msg=k)
    for L, c in zip(rest, caches[1:]):
        want = O.cache_from_hidden(L, pre["h2"], 32)
        np.testing.assert_array_equal(c.K[:, :20], want.K[:, :20])
        np.testing.assert_array_equal(c.V[:, :20], want.V[:, :20])


def test_block_candidates_are_independent_at_depth():
    layers = _stack(MINI, 60, 3)
    W, D = 3, 4
    ctx = synth.uniform_tokens(61, 22, MINI.vocab)
    cand = synth.uniform_tokens(61, W * D, MINI.vocab, stream=1)
    base = O.stack_prefill(layers, ctx, 48)
    blk = O.stack_span_forward(layers, [c.copy() for c in base], cand, mode="block", W=W, D=D, commit=False)
    for w in range(W):
        one = O.stack_span_forward(layers, [c.copy() for c in base], cand[w * D:(w + 1) * D])
        rows = slice(w * D, (w + 1) * D)
        for k in ("hidden_out", "logits"):
            np.testing.assert_allclose(blk[k][rows], one[k], rtol=0, atol=0, err_msg=f"w={w} {k}")
