"""GPU parity of the full-depth stack call (cad_stack_span_forward) against the oracle's stack.

Rounding drift between an fp32-accumulating pipeline and the fp64 oracle enters every layer
independently (bf16 rounding flips of the normed inputs and the SwiGLU product), so the
one-layer tolerances are widened by sqrt(depth) for outputs after the last layer and by
sqrt(l + 1) for the K/V rows of layer l."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from spec_verify_cad_amd import cad, synth
from spec_verify_cad_amd.configs import SMALL

from gpu_util import argmax_check, hidden_tol, log, logit_tol, to_f64
from helpers import oracle_layer

pytestmark = pytest.mark.gpu

NL = 4


def _stack_weights(shape, seed, n):
    out = []
    for l in range(n):
        names = [k for k in synth.weight_shapes(shape)
                 if not (k == "embed" and l > 0) and not (k == "w_lm" and l < n - 1)]
        out.append(synth.layer_weights(shape, seed + l, names=names))
    return out


@pytest.fixture(scope="module")
def small_stack():
    ws = _stack_weights(SMALL, 300, NL)
    dst = cad.DeviceStack([cad.DeviceLayer(SMALL, w) for w in ws])
    ols = [oracle_layer(SMALL, w, only=list(w)) for w in ws]
    return ws, dst, ols


def _prefill(dst, sc, ctx, chunk=64):
    for s in range(0, ctx.shape[1], chunk):
        t = torch.from_numpy(np.ascontiguousarray(ctx[:, s:s + chunk], dtype=np.int32)).cuda()
        cad.stack_span_forward(dst, sc, t, t.shape[1], flags=cad.KV_ONLY | cad.COMMIT_ALL)


def _run(dst, sc, toks, mode=cad.MASK_CAUSAL, W=1, D=1, flags=0):
    B, Nq = toks.shape
    s = dst.shape
    t = torch.from_numpy(np.ascontiguousarray(toks, dtype=np.int32)).cuda()
    last = bool(flags & cad.LOGITS_LAST)
    R = B if last else B * Nq
    am = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    hid = torch.zeros((B * Nq, s.hidden), dtype=torch.int16, device="cuda")
    lg = torch.zeros((R, s.vocab), dtype=torch.float32, device="cuda")
    cad.stack_span_forward(dst, sc, t, Nq, mode, W, D, flags, am, hid, lg)
    torch.cuda.synchronize()
    return am.cpu().numpy(), to_f64(hid, "bf16"), lg.cpu().numpy().astype(np.float64)


def _check_out(g_a, g_h, g_l, ref, rows, n_layers, what):
    href = ref["hidden_out"]
    dh = np.abs(g_h - href)
    scale = math.sqrt(n_layers)
    tol_h = np.maximum(hidden_tol(href, SMALL.ffn) * scale, hidden_tol(href, SMALL.ffn))
    assert (dh <= tol_h).all(), f"{what} hidden max-abs {dh.max():.3e}"
    ltol = logit_tol(SMALL.hidden) * scale
    dl = np.abs(g_l - ref["logits"]).max()
    assert dl <= ltol, f"{what} logits max-abs {dl:.3e} > {ltol:.3g}"
    unique = argmax_check(g_a, ref, g_l, what, ltol)
    log(f"{what}: hidden {dh.max():.3e} logits {dl:.3e} (tol {ltol:.3g}) unique argmax {int(unique.sum())}/{len(g_a)}")


def _check_caches(sc, b, ocs, lo, hi, what):
    for l, oc in enumerate(ocs):
        k = to_f64(sc.caches[l].k[b, :, lo:hi], "bf16")
        v = to_f64(sc.caches[l].v[b, :, :, lo:hi], "bf16").transpose(0, 2, 1)
        for name, got, ref in (("k", k, oc.K[:, lo:hi]), ("v", v, oc.V[:, lo:hi])):
            d = np.abs(got - ref)
            tol = hidden_tol(ref) * math.sqrt(l + 1)
            frac = float(np.mean(d > 0))
            assert (d <= tol).all(), f"{what} layer {l} {name} max-abs {d.max():.3e}"
            log(f"{what} layer {l} {name}: max-abs {d.max():.3e}, differing {frac:.4f}")


@pytest.mark.parametrize("Nq", [1, 13, 70])
def test_small_stack_span_matches_oracle(small_stack, Nq):
    ws, dst, ols = small_stack
    log(f"stack of {NL} small layers, causal Nq={Nq}")
    B, L0, cap = 2, 100, 192
    ctx = np.stack([synth.uniform_tokens(310 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(320 + b, Nq, SMALL.vocab) for b in range(B)])
    sc = cad.StackCache(SMALL, NL, B, cap)
    _prefill(dst, sc, ctx)
    assert list(sc.len.cpu().numpy()) == [L0] * B
    g_a, g_h, g_l = _run(dst, sc, span, flags=cad.COMMIT_ALL)
    assert list(sc.len.cpu().numpy()) == [L0 + Nq] * B
    for b in range(B):
        ocs = O.stack_prefill(ols, ctx[b], cap, chunk=64)
        _check_caches(sc, b, ocs, 0, L0, f"prefill b={b}")
        ref = O.stack_span_forward(ols, ocs, span[b])
        rows = slice(b * Nq, (b + 1) * Nq)
        _check_out(g_a[rows], g_h[rows], g_l[rows], ref, rows, NL, f"b={b}")
        _check_caches(sc, b, ocs, L0, L0 + Nq, f"span b={b}")


def test_small_stack_block_verify_and_copy_commit(small_stack):
    ws, dst, ols = small_stack
    W, D, B, L0, cap = 3, 4, 2, 80, 128
    log("stack block W=3 D=4, then copy-commit Nq=9")
    ctx = np.stack([synth.uniform_tokens(330 + b, L0, SMALL.vocab) for b in range(B)])
    cand = np.stack([synth.uniform_tokens(340 + b, W * D, SMALL.vocab) for b in range(B)])
    sc = cad.StackCache(SMALL, NL, B, cap)
    _prefill(dst, sc, ctx)
    g_a, g_h, g_l = _run(dst, sc, cand, mode=cad.MASK_BLOCK, W=W, D=D)
    assert list(sc.len.cpu().numpy()) == [L0] * B                 # verify forward: no commit
    ocs = [O.stack_prefill(ols, ctx[b], cap, chunk=64) for b in range(B)]
    for b in range(B):
        ref = O.stack_span_forward(ols, [c.copy() for c in ocs[b]], cand[b], mode="block", W=W, D=D, commit=False)
        rows = slice(b * W * D, (b + 1) * W * D)
        _check_out(g_a[rows], g_h[rows], g_l[rows], ref, rows, NL, f"block b={b}")
    # copy-commit mode through the stack: the LM head for each sequence's last row only
    Nq = 9
    span = np.stack([synth.uniform_tokens(350 + b, Nq, SMALL.vocab) for b in range(B)])
    g_a, g_h, g_l = _run(dst, sc, span, flags=cad.COMMIT_ALL | cad.LOGITS_LAST)
    assert list(sc.len.cpu().numpy()) == [L0 + Nq] * B
    for b in range(B):
        ref = O.stack_span_forward(ols, ocs[b], span[b])
        last = {k: ref[k][Nq - 1:Nq] for k in ("logits", "argmax", "top2_gap")}
        last["hidden_out"] = ref["hidden_out"]
        dh = np.abs(g_h[b * Nq:(b + 1) * Nq] - ref["hidden_out"])
        assert (dh <= hidden_tol(ref["hidden_out"], SMALL.ffn) * math.sqrt(NL)).all()
        dl = np.abs(g_l[b:b + 1] - last["logits"]).max()
        assert dl <= logit_tol(SMALL.hidden) * math.sqrt(NL)
        argmax_check(g_a[b:b + 1], last, g_l[b:b + 1], f"copy-commit b={b}", logit_tol(SMALL.hidden) * math.sqrt(NL))
        _check_caches(sc, b, ocs[b], L0, L0 + Nq, f"copy-commit b={b}")


def test_one_layer_stack_is_bitwise_the_one_layer_call(small_stack):
    ws, dst, ols = small_stack
    # a one-layer stack: its only layer carries the embedding and the LM head
    lay = cad.DeviceLayer(SMALL, synth.layer_weights(SMALL, 300))
    one = cad.DeviceStack([lay])
    B, L0, cap, Nq = 2, 50, 96, 11
    ctx = np.stack([synth.uniform_tokens(360 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(370 + b, Nq, SMALL.vocab) for b in range(B)])
    sc = cad.StackCache(SMALL, 1, B, cap)
    c1 = cad.DeviceCache(SMALL, B, cap)
    _prefill(one, sc, ctx)
    for s in range(0, L0, 64):
        t = torch.from_numpy(np.ascontiguousarray(ctx[:, s:s + 64], dtype=np.int32)).cuda()
        cad.span_forward(lay, c1, t, t.shape[1], flags=cad.KV_ONLY | cad.COMMIT_ALL)
    a = _run(one, sc, span, flags=cad.COMMIT_ALL)
    t = torch.from_numpy(np.ascontiguousarray(span, dtype=np.int32)).cuda()
    am = torch.full((B * Nq,), -7, dtype=torch.int32, device="cuda")
    hid = torch.zeros((B * Nq, SMALL.hidden), dtype=torch.int16, device="cuda")
    lg = torch.zeros((B * Nq, SMALL.vocab), dtype=torch.float32, device="cuda")
    cad.span_forward(lay, c1, t, Nq, flags=cad.COMMIT_ALL, argmax_out=am, hidden_out=hid, logits_out=lg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a[0], am.cpu().numpy())
    np.testing.assert_array_equal(a[2], lg.cpu().numpy())
    np.testing.assert_array_equal(sc.caches[0].k.cpu().numpy(), c1.k.cpu().numpy())
    np.testing.assert_array_equal(sc.caches[0].v.cpu().numpy(), c1.v.cpu().numpy())


def test_stack_argument_errors(small_stack):
    ws, dst, ols = small_stack
    sc = cad.StackCache(SMALL, NL, 1, 64)
    t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    am = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        cad.stack_span_forward(dst, cad.StackCache(SMALL, NL - 1, 1, 64), t, 4, argmax_out=am)
    L = cad.lib()
    ws_ = cad.alloc_workspace(1 << 24)
    import ctypes
    assert L.cad_stack_span_forward(dst.descs, 0, sc.descs, ctypes.c_void_p(t.data_ptr()), 1, 4, 0, 1, 1, 0,
                                    ctypes.c_void_p(am.data_ptr()), None, None, ctypes.c_void_p(ws_.data_ptr()),
                                    ws_.numel(), None) == cad.CAD_EINVAL
    # a layer of another shape in the stack
    other = cad.DeviceLayer(synth.LayerShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                                             vocab=SMALL.vocab),
                            synth.layer_weights(synth.LayerShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                                                 ffn=512, vocab=SMALL.vocab), 9))
    mixed = cad.DeviceStack(dst.layers[:NL - 1] + [other])
    with pytest.raises(cad.CadError):
        cad.stack_span_forward(mixed, sc, t, 4, argmax_out=am, workspace=ws_)
    torch.cuda.synchronize()
    assert int(sc.len[0]) == 0


def test_full_depth_1p5b_stack_matches_oracle():
    """The 28-layer stack of the 1.5B shape the full-depth curve times: a 64-token prefix, an
    8-token span (all rows' logits), then a copy-commit span, against the oracle's stack."""
    from spec_verify_cad_amd.configs import QWEN15
    nl, L0, cap, N = 28, 64, 96, 8
    log("full-depth 1.5B stack: weights")
    ws = _stack_weights(QWEN15, 900, nl)
    dst = cad.DeviceStack([cad.DeviceLayer(QWEN15, w) for w in ws])
    log("full-depth 1.5B stack: oracle weights")
    ols = [oracle_layer(QWEN15, w, only=list(w)) for w in ws]
    del ws
    ctx = synth.uniform_tokens(910, L0, QWEN15.vocab)[None]
    span = synth.uniform_tokens(911, 2 * N, QWEN15.vocab)[None]
    sc = cad.StackCache(QWEN15, nl, 1, cap)
    _prefill(dst, sc, ctx, chunk=64)
    t = torch.from_numpy(np.ascontiguousarray(span[:, :N], dtype=np.int32)).cuda()
    am = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    hid = torch.zeros((N, QWEN15.hidden), dtype=torch.int16, device="cuda")
    lg = torch.zeros((N, QWEN15.vocab), dtype=torch.float32, device="cuda")
    cad.stack_span_forward(dst, sc, t, N, flags=cad.COMMIT_ALL, argmax_out=am, hidden_out=hid, logits_out=lg)
    t2 = torch.from_numpy(np.ascontiguousarray(span[:, N:], dtype=np.int32)).cuda()
    am2 = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    lg2 = torch.zeros((1, QWEN15.vocab), dtype=torch.float32, device="cuda")
    cad.stack_span_forward(dst, sc, t2, N, flags=cad.COMMIT_ALL | cad.LOGITS_LAST, argmax_out=am2, logits_out=lg2)
    torch.cuda.synchronize()
    assert int(sc.len[0]) == L0 + 2 * N
    log("full-depth 1.5B stack: oracle prefill and spans")
    ocs = O.stack_prefill(ols, ctx[0], cap, chunk=64)
    ref = O.stack_span_forward(ols, ocs, span[0, :N])
    scale = math.sqrt(nl)
    g_h = to_f64(hid, "bf16")
    dh = np.abs(g_h - ref["hidden_out"])
    tol_h = hidden_tol(ref["hidden_out"], QWEN15.ffn) * scale
    ltol = logit_tol(QWEN15.hidden) * scale
    g_l = lg.cpu().numpy().astype(np.float64)
    dl = np.abs(g_l - ref["logits"]).max()
    log(f"28 layers: hidden max-abs {dh.max():.3e} (tol from {tol_h.min():.3g}), logits max-abs {dl:.3e} (tol {ltol:.3g})")
    assert (dh <= tol_h).all()
    assert dl <= ltol
    argmax_check(am.cpu().numpy(), ref, g_l, "28-layer span", ltol)
    ref2 = O.stack_span_forward(ols, ocs, span[0, N:])
    last = {k: ref2[k][N - 1:N] for k in ("logits", "argmax", "top2_gap")}
    g_l2 = lg2.cpu().numpy().astype(np.float64)
    assert np.abs(g_l2 - last["logits"]).max() <= ltol
    argmax_check(am2.cpu().numpy(), last, g_l2, "28-layer copy-commit", ltol)
    # the first and last layers' cache rows of the whole sequence
    for l in (0, nl - 1):
        k_ = to_f64(sc.caches[l].k[0, :, :L0 + 2 * N], "bf16")
        d = np.abs(k_ - ocs[l].K[:, :L0 + 2 * N])
        assert (d <= hidden_tol(ocs[l].K[:, :L0 + 2 * N]) * math.sqrt(l + 1)).all(), f"layer {l} K {d.max()}"
        log(f"layer {l} K rows: max-abs {d.max():.3e}")


def test_tiny_fp32_stack_matches_oracle():
    """A 3-layer stack of the tiny fp32 layer (the simple attention path) against the oracle."""
    from spec_verify_cad_amd.configs import TINY
    nl, L0, cap, N = 3, 40, 64, 8
    ws = _stack_weights(TINY, 500, nl)
    dst = cad.DeviceStack([cad.DeviceLayer(TINY, w) for w in ws])
    ols = [oracle_layer(TINY, w, only=list(w)) for w in ws]
    ctx = synth.uniform_tokens(510, L0, TINY.vocab)[None]
    span = synth.uniform_tokens(511, N, TINY.vocab)[None]
    sc = cad.StackCache(TINY, nl, 1, cap)
    _prefill(dst, sc, ctx)
    t = torch.from_numpy(np.ascontiguousarray(span, dtype=np.int32)).cuda()
    am = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    hid = torch.zeros((N, TINY.hidden), dtype=torch.float32, device="cuda")
    lg = torch.zeros((N, TINY.vocab), dtype=torch.float32, device="cuda")
    cad.stack_span_forward(dst, sc, t, N, flags=cad.COMMIT_ALL, argmax_out=am, hidden_out=hid, logits_out=lg)
    torch.cuda.synchronize()
    ocs = O.stack_prefill(ols, ctx[0], cap)
    ref = O.stack_span_forward(ols, ocs, span[0])
    dh = np.abs(hid.cpu().numpy().astype(np.float64) - ref["hidden_out"]).max()
    g_l = lg.cpu().numpy().astype(np.float64)
    dl = np.abs(g_l - ref["logits"]).max()
    log(f"tiny fp32 stack: hidden {dh:.3e} logits {dl:.3e}")
    assert dh <= 1e-4 and dl <= 1e-4
    argmax_check(am.cpu().numpy(), ref, g_l, "tiny fp32 stack", 1e-4)
    for l in range(nl):
        k_ = sc.caches[l].k[0, :, :L0 + N].cpu().numpy().astype(np.float64)
        assert np.abs(k_ - ocs[l].K[:, :L0 + N]).max() <= 1e-4


def test_small_stack_cad_program_matches_oracle():
    """A short Copy-as-Decode program with its op-boundary steps through a 3-layer stack (the
    vocabulary holds the grammar's token ids): every decision against the oracle's stack, and
    every layer's cache at the end."""
    from spec_verify_cad_amd.program import DeviceProgram
    shp = synth.LayerShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=704, vocab=15013)
    nl = 3
    ws = _stack_weights(shp, 700, nl)
    dst = cad.DeviceStack([cad.DeviceLayer(shp, w) for w in ws])
    ols = [oracle_layer(shp, w, only=list(w)) for w in ws]
    doc = synth.uniform_tokens(710, 300, shp.vocab)
    ops = [("copy", 10, 25), ("gen", 3), ("copy", 150, 40), ("gen", 2), ("copy", 0, 7)]
    fwds = synth.cad_program_forwards(ops)
    fed = sum(f.n for f in fwds)
    cap = ((len(doc) + fed + 8 + 3) // 4) * 4
    sc = cad.StackCache(shp, nl, 1, cap)
    _prefill(dst, sc, doc[None], chunk=128)
    prog = DeviceProgram(dst, sc, doc, fwds)
    log(f"stack program: {len(fwds)} forwards, {fed} fed tokens")
    prog.enqueue()
    torch.cuda.synchronize()
    assert int(sc.len[0]) == len(doc) + fed
    dec = prog.decisions.cpu().numpy()
    stream = prog.fed_tokens(doc)
    ocs = O.stack_prefill(ols, doc, cap, chunk=128)
    tol = logit_tol(shp.hidden) * math.sqrt(nl)
    pos, firm = 0, 0
    for f, pf in enumerate(fwds):
        ref = O.stack_span_forward(ols, ocs, stream[pos:pos + pf.n])
        last = {k: ref[k][-1:] for k in ("logits", "argmax", "top2_gap")}
        if pf.allowed is None:
            argmax_check(dec[f:f + 1], last, None, f"forward {f} ({pf.role})", tol)
        else:
            assert int(dec[f]) in pf.allowed
            best, _, gap = O.masked_argmax(last["logits"], np.asarray([pf.allowed]), shp.vocab)
            if gap[0] > 2 * tol:
                firm += 1
                assert dec[f] == best[0], f"forward {f} ({pf.role}): {dec[f]} vs {best[0]}"
        pos += pf.n
    log(f"stack program: {firm} masked decisions firm")
    for l in range(nl):
        k_ = to_f64(sc.caches[l].k[0, :, :len(doc) + fed], "bf16")
        d = np.abs(k_ - ocs[l].K[:, :len(doc) + fed])
        assert (d <= hidden_tol(ocs[l].K[:, :len(doc) + fed]) * math.sqrt(l + 1)).all(), f"layer {l}"


def test_small_stack_sampled_verify_matches_oracle(small_stack):
    """Stochastic verification through the 4-layer small stack: a greedy-chain draft at a small
    temperature (drafts kept) and a random draft, against the oracle's stack and draws."""
    ws, dst, ols = small_stack
    B, L0, cap, k, T, seed = 2, 70, 128, 6, 0.05, 4242
    Nq = k + 1
    ctx = np.stack([synth.uniform_tokens(720 + b, L0, SMALL.vocab) for b in range(B)])
    g = [int(x) for x in synth.uniform_tokens(730, B, SMALL.vocab)]
    chain, c = [], O.stack_prefill(ols, ctx[0], cap)
    t = g[0]
    for _ in range(k):
        t = int(O.stack_decode_one(ols, c, t)["argmax"][0])
        chain.append(t)
    toks = np.array([[g[0]] + chain, [g[1]] + list(synth.uniform_tokens(731, k, SMALL.vocab))], dtype=np.int32)
    dls = [k, 4]
    sc = cad.StackCache(SMALL, NL, B, cap)
    _prefill(dst, sc, ctx)
    pred = torch.full((B * Nq,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros((B * Nq, SMALL.vocab), dtype=torch.float32, device="cuda")
    T32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    cad.stack_span_forward_sampled(dst, sc, T32(toks), Nq, T, seed, draft_len=T32(dls), pred_out=pred, logits_out=lg)
    torch.cuda.synchronize()
    g_pred, g_l = pred.cpu().numpy(), lg.cpu().numpy().astype(np.float64)
    kept = 0
    for b in range(B):
        ref = O.stack_span_forward(ols, O.stack_prefill(ols, ctx[b], cap), toks[b], commit=False)
        rows = slice(b * Nq, (b + 1) * Nq)
        opred = O.sampled_predictions(ref["logits"], toks[b], dls[b], T, seed, b, L0)[0]
        y_gap, z_gap, acc_m = O.sampled_margins(ref["logits"], toks[b], dls[b], T, seed, b, L0)
        e = np.max(np.abs(g_l[rows] - ref["logits"]), axis=1)
        for i in range(Nq):
            m = 2 * e[i] / T + 1e-6
            firm = (acc_m[i] > math.expm1(m) and (opred[i] == toks[b, i + 1] or z_gap[i] > m)) if i < dls[b] \
                else y_gap[i] > m
            if firm:
                assert g_pred[rows][i] == opred[i], (b, i, g_pred[rows][i], opred[i])
        kept += sum(1 for i in range(dls[b]) if opred[i] == toks[b, i + 1])
    assert kept >= 1
