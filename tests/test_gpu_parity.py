"""GPU parity of the three C-ABI calls against the CPU oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as O
from spec_verify_cad_amd import cad, synth
from spec_verify_cad_amd.configs import CONFIGS, SMALL, TINY
from spec_verify_cad_amd.synth import LayerShape

from gpu_util import (LOGIT_TOL, NEAR_TIE, argmax_check, compare, compare_cache, hidden_tol, log, prefill, run_forward, to_f64,
                      upload_oracle_cache)
from helpers import oracle_layer

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------- n-gram lookup
def _lookup_gpu(ctx_list, n, W, D, with_current, stride=None):
    B = len(ctx_list)
    stride = stride or max(max(len(c) for c in ctx_list), 1)
    ctx = np.zeros((B, stride), dtype=np.int32)
    for b, c in enumerate(ctx_list):
        ctx[b, :len(c)] = c
    lens = np.array([len(c) for c in ctx_list], dtype=np.int32)
    tc, tl = torch.from_numpy(ctx).cuda(), torch.from_numpy(lens).cuda()
    draft = torch.full((B, with_current + W * D), -9, dtype=torch.int32, device="cuda")
    dlen = torch.full((B, W), -9, dtype=torch.int32, device="cuda")
    mpos = torch.full((B, W), -9, dtype=torch.int32, device="cuda")
    cad.ngram_lookup(tc, tl, n, W, D, with_current, draft, dlen, mpos)
    torch.cuda.synchronize()
    return draft.cpu().numpy(), dlen.cpu().numpy(), mpos.cpu().numpy()


@pytest.mark.parametrize("n,W,D,wc", [(1, 1, 4, 0), (2, 3, 5, 1), (3, 1, 10, 1), (5, 4, 8, 0), (4, 8, 64, 0)])
def test_ngram_lookup_matches_oracle_small_alphabets(n, W, D, wc):
    log(f"ngram small n={n} W={W} D={D} wc={wc}")
    rng = np.random.default_rng(100 + n)
    ctxs = [rng.integers(0, 3, size=int(rng.integers(0, 700))) for _ in range(48)]
    ctxs += [np.zeros(0, np.int64), np.array([1]), np.array([2, 2]), np.full(600, 5)]
    d, l, m = _lookup_gpu(ctxs, n, W, D, wc)
    for b, c in enumerate(ctxs):
        od, ol, om = O.ngram_lookup(c, len(c), n, W, D)
        np.testing.assert_array_equal(l[b], ol, err_msg=f"b={b}")
        np.testing.assert_array_equal(m[b], om, err_msg=f"b={b}")
        np.testing.assert_array_equal(d[b, wc:].reshape(W, D), od, err_msg=f"b={b}")
        if wc:
            assert d[b, 0] == (c[-1] if len(c) else 0)


@pytest.mark.parametrize("n,W", [(3, 1), (5, 4)])
def test_ngram_lookup_matches_in_the_oldest_chunk(n, W):
    # histories of several 8192-start scan chunks whose only matches sit at the very start, so the
    # scan runs to the oldest chunk (window positions before 0, the next window fetched past the
    # end); plus a history shorter than one chunk and one of exactly n + 1 tokens
    log(f"ngram oldest-chunk matches n={n} W={W}")
    rng = np.random.default_rng(300 + n)
    V = 1 << 30                                        # ids drawn from 2^30: no accidental matches
    ctxs = []
    for L in (8192 + n + 1, 8192 + n + 2, 20000, 3 * 8192 + 11, 5000):
        c = rng.integers(0, V, size=L)
        c[L - n:] = [7, 8, 9, 10, 11][:n]              # the suffix
        for j in range(min(W, 3)):                     # planted at starts 0, 1, 2 (overlapping)
            c[j:j + n] = c[L - n:]
        ctxs.append(c)
    ctxs.append(np.array([7, 8, 9, 10, 11, 12][:n + 1]))
    d, l, m = _lookup_gpu(ctxs, n, W, 6, 0)
    for b, c in enumerate(ctxs):
        od, ol, om = O.ngram_lookup(c, len(c), n, W, 6)
        np.testing.assert_array_equal(l[b], ol, err_msg=f"b={b}")
        np.testing.assert_array_equal(m[b], om, err_msg=f"b={b}")
        np.testing.assert_array_equal(d[b].reshape(W, 6), od, err_msg=f"b={b}")
    assert (m[:5, 0] >= 0).all()                       # the planted starts are found


def test_ngram_lookup_planted_contexts():
    # contexts shaped like the batched PLD workload (Zipf background, planted copies), n=3, D=10
    log("ngram planted zipf contexts")
    ctxs = [synth.planted_context(7, 4000 + 37 * b, 50000, 0.4, 8, 256, "zipf", 1.1, stream=b)[0] for b in range(16)]
    d, l, m = _lookup_gpu(ctxs, 3, 1, 10, 1)
    for b, c in enumerate(ctxs):
        od, ol, om = O.ngram_lookup(c, len(c), 3, 1, 10)
        assert m[b, 0] == om[0] and l[b, 0] == ol[0]
        np.testing.assert_array_equal(d[b, 1:], od[0])


@pytest.mark.parametrize("n_max,n_min,W,D,wc", [(3, 1, 1, 10, 1), (4, 2, 3, 5, 0), (6, 1, 8, 8, 0)])
def test_ngram_lookup_longest_matches_oracle(n_max, n_min, W, D, wc):
    log(f"ngram longest n={n_max}..{n_min} W={W} D={D}")
    rng = np.random.default_rng(200 + n_max)
    ctxs = [rng.integers(0, 4, size=int(rng.integers(0, 900))) for _ in range(40)]
    ctxs += [np.zeros(0, np.int64), np.array([3]), np.array([1, 2, 3, 4, 5])]
    ctxs += [synth.planted_context(9, 6000 + 11 * b, 50000, 0.4, 8, 256, "zipf", 1.1, stream=b)[0] for b in range(8)]
    B = len(ctxs)
    stride = max(len(c) for c in ctxs)
    ctx = np.zeros((B, stride), dtype=np.int32)
    for b, c in enumerate(ctxs):
        ctx[b, :len(c)] = c
    tc = torch.from_numpy(ctx).cuda()
    tl = torch.from_numpy(np.array([len(c) for c in ctxs], dtype=np.int32)).cuda()
    draft = torch.full((B, wc + W * D), -9, dtype=torch.int32, device="cuda")
    dlen = torch.full((B, W), -9, dtype=torch.int32, device="cuda")
    mpos = torch.full((B, W), -9, dtype=torch.int32, device="cuda")
    mn = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    cad.ngram_lookup_longest(tc, tl, n_max, n_min, W, D, wc, draft, dlen, mpos, mn)
    torch.cuda.synchronize()
    d, l, m, nn = (t.cpu().numpy() for t in (draft, dlen, mpos, mn))
    for b, c in enumerate(ctxs):
        od, ol, om, on = O.ngram_lookup_longest(c, len(c), n_max, n_min, W, D)
        assert nn[b] == on, f"b={b}"
        np.testing.assert_array_equal(l[b], ol, err_msg=f"b={b}")
        np.testing.assert_array_equal(m[b], om, err_msg=f"b={b}")
        np.testing.assert_array_equal(d[b, wc:].reshape(W, D), od, err_msg=f"b={b}")


# ------------------------------------------------------------------------- accept scan
def test_accept_scan_causal_matches_oracle():
    log("accept causal")
    rng = np.random.default_rng(5)
    B, D, V = 300, 10, 3
    g = rng.integers(0, V, size=(B, 1))
    drafts = rng.integers(0, V, size=(B, D))
    dl = rng.integers(0, D + 1, size=(B, 1))
    pred = rng.integers(0, V, size=(B, 1 + D))
    for b in range(0, B, 3):                       # plant long agreements
        k = int(rng.integers(0, D + 1))
        pred[b, :k] = drafts[b, :k]
    rows = np.concatenate([g, drafts], axis=1).astype(np.int32)
    ctx_cap = 64
    ctx = np.zeros((B, ctx_cap), dtype=np.int32)
    clen = rng.integers(0, 30, size=B).astype(np.int32)
    cache = cad.DeviceCache(SMALL, B, 128)
    kvlen = rng.integers(0, 100, size=B).astype(np.int32)
    cache.len.copy_(torch.from_numpy(kvlen))
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out = [torch.full((B,), -1, dtype=torch.int32, device="cuda") for _ in range(3)]
    em = torch.full((B, D + 1), -1, dtype=torch.int32, device="cuda")
    tctx, tclen = T(ctx), T(clen)
    cad.accept_scan(T(rows), 1, T(dl), T(pred), None, B, 1, D, cad.MASK_CAUSAL, out[0], out[1], em, out[2],
                    ctx=tctx, ctx_len=tclen, ctx_cap=ctx_cap, cache=cache)
    torch.cuda.synchronize()
    acc, bw, ne = (o.cpu().numpy() for o in out)
    emn, ctxn, clenn, kvn = em.cpu().numpy(), tctx.cpu().numpy(), tclen.cpu().numpy(), cache.len.cpu().numpy()
    for b in range(B):
        a, e = O.accept_causal(drafts[b], int(dl[b, 0]), pred[b])
        assert acc[b] == a and ne[b] == a + 1 and bw[b] == 0
        assert list(emn[b, :a + 1]) == e and not emn[b, a + 1:].any()
        assert list(ctxn[b, clen[b]:clen[b] + a + 1]) == e and clenn[b] == clen[b] + a + 1
        assert kvn[b] == kvlen[b] + a + 1


def test_accept_scan_block_with_row_compaction():
    log("accept block + compaction")
    rng = np.random.default_rng(6)
    shp = SMALL
    B, W, D, V, cap = 24, 4, 8, 3, 96
    drafts = rng.integers(0, V, size=(B, W, D))
    dl = rng.integers(0, D + 1, size=(B, W))
    pred = rng.integers(0, V, size=(B, W * D))
    fp = rng.integers(0, V, size=B)
    for b in range(B):
        w = int(rng.integers(0, W))
        k = int(rng.integers(0, D + 1))
        seq = [fp[b]] + list(pred[b, w * D:(w + 1) * D - 1])
        drafts[b, w, :k] = seq[:k]
        dl[b, w] = max(dl[b, w], k)
    cache = cad.DeviceCache(shp, B, cap)
    kvlen = rng.integers(0, cap - W * D, size=B).astype(np.int32)
    cache.len.copy_(torch.from_numpy(kvlen))
    kinit = torch.randint(-30000, 30000, cache.k.shape, dtype=torch.int16, device="cuda")
    vinit = torch.randint(-30000, 30000, cache.v.shape, dtype=torch.int16, device="cuda")
    cache.k.copy_(kinit)
    cache.v.copy_(vinit)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    acc, bw, ne = (torch.full((B,), -1, dtype=torch.int32, device="cuda") for _ in range(3))
    em = torch.full((B, D + 1), -1, dtype=torch.int32, device="cuda")
    cad.accept_scan(T(drafts.reshape(B, -1)), 0, T(dl), T(pred), T(fp), B, W, D, cad.MASK_BLOCK, acc, bw, em, ne,
                    cache=cache)
    torch.cuda.synchronize()
    K0, V0, K1, V1 = kinit.cpu().numpy(), vinit.cpu().numpy(), cache.k.cpu().numpy(), cache.v.cpu().numpy()
    for b in range(B):
        a, w, e, _ = O.accept_block(drafts[b], dl[b], pred[b], int(fp[b]), D)
        assert acc[b].item() == a and bw[b].item() == w and ne[b].item() == a + 1
        assert list(em[b, :a + 1].cpu().numpy()) == e
        L = int(kvlen[b])
        assert cache.len[b].item() == L + a
        want_k, want_v = K0[b].copy(), V0[b].copy()
        want_k[:, L:L + a] = K0[b][:, L + w * D:L + w * D + a]
        want_v[:, :, L:L + a] = V0[b][:, :, L + w * D:L + w * D + a]      # v is dim-major [g, d, slot]
        np.testing.assert_array_equal(K1[b], want_k)
        np.testing.assert_array_equal(V1[b], want_v)


# ------------------------------------------------------------------------- span forward
@pytest.fixture(scope="module")
def small():
    w = synth.layer_weights(SMALL, 77)
    return w, cad.DeviceLayer(SMALL, w), oracle_layer(SMALL, w)


def test_tiny_fp32_span_matches_oracle_and_decode_steps():
    wl = CONFIGS["tiny_f32"]
    log("tiny fp32 span vs oracle")
    w = synth.layer_weights(TINY, wl.seed)
    OL = oracle_layer(TINY, w)
    oc = O.cache_from_hidden(OL, synth.hidden_states(wl.seed, wl.cache_len, TINY.hidden), 160)
    span = synth.uniform_tokens(wl.seed, 8, TINY.vocab, stream=1)
    ref = O.span_forward(OL, oc.copy(), span)
    dl = cad.DeviceLayer(TINY, w)
    cache = cad.DeviceCache(TINY, 1, 160)
    upload_oracle_cache(cache, 0, oc, "f32")
    g = run_forward(dl, cache, span[None], flags=cad.COMMIT_ALL)
    compare(g, ref, what="tiny span")
    assert cache.len.item() == 136
    # the same 8 tokens as 8 single-token forwards on the GPU
    c2 = cad.DeviceCache(TINY, 1, 160)
    upload_oracle_cache(c2, 0, oc, "f32")
    steps = [run_forward(dl, c2, np.array([[t]]), flags=cad.COMMIT_ALL) for t in span]
    g2 = {k: np.concatenate([s[k] for s in steps]) for k in ("argmax", "hidden", "logits")}
    compare(g2, ref, what="tiny decode steps")
    assert np.max(np.abs(g2["hidden"] - g["hidden"])) <= 1e-5


def test_tiny_fp32_corrupted_draft_accepts_four():
    wl = CONFIGS["tiny_f32"]
    log("tiny fp32 a=4")
    w = synth.layer_weights(TINY, wl.seed)
    OL = oracle_layer(TINY, w)
    oc = O.cache_from_hidden(OL, synth.hidden_states(wl.seed, wl.cache_len, TINY.hidden), 160)
    span = synth.uniform_tokens(wl.seed, 8, TINY.vocab, stream=1)
    g = int(span[0])
    c = oc.copy()
    greedy = []
    t = g
    for _ in range(8):
        t = int(O.decode_one(OL, c, t)["argmax"][0])
        greedy.append(t)
    draft = np.array(greedy)
    draft[4] = (draft[4] + 1) % TINY.vocab
    dl = cad.DeviceLayer(TINY, w)
    cache = cad.DeviceCache(TINY, 1, 160)
    upload_oracle_cache(cache, 0, oc, "f32")
    rows = np.concatenate([[g], draft])[None].astype(np.int32)
    res = run_forward(dl, cache, rows)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    acc, bw, ne = (torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(3))
    em = torch.zeros((1, 9), dtype=torch.int32, device="cuda")
    cad.accept_scan(T(rows), 1, T([[8]]), T(res["argmax"][None]), None, 1, 1, 8, cad.MASK_CAUSAL, acc, bw, em, ne,
                    cache=cache)
    torch.cuda.synchronize()
    assert acc.item() == 4 and ne.item() == 5
    assert list(em[0, :5].cpu().numpy()) == greedy[:5]
    assert cache.len.item() == 128 + 5


@pytest.mark.parametrize("Nq", [1, 8, 13, 17, 20, 40, 100])
def test_small_bf16_span_matches_oracle(small, Nq):
    # Nq = 17 and 20: 68 and 80 rows per GQA group (4 query heads), the two-key-phase attention tile
    w, dl, OL = small
    log(f"small bf16 causal Nq={Nq}")
    B, L0, cap = 3, 150, 320
    ctx = np.stack([synth.uniform_tokens(50 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(60 + b, Nq, SMALL.vocab) for b in range(B)])
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx, chunk=64)
    g = run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
    assert list(cache.len.cpu().numpy()) == [L0 + Nq] * B
    for b in range(B):
        oc = O.cache_from_tokens(OL, ctx[b], cap)
        compare_cache(cache, b, oc, 0, L0, "bf16", what=f"prefill b={b}")
        ref = O.span_forward(OL, oc, span[b])
        compare(g, ref, rows=slice(b * Nq, (b + 1) * Nq), what=f"b={b}")
        compare_cache(cache, b, oc, L0, L0 + Nq, "bf16", what=f"span rows b={b}")


@pytest.mark.parametrize("B, Nq", [(3, 12), (3, 40), (1, 97), (3, 100)])
def test_small_bf16_lm_head_without_logits_matches_oracle(small, B, Nq):
    # 33..128 LM-head rows run on balanced vocabulary ranges (the 5003-id vocabulary makes short
    # last chunks), 300 rows on 256 x 256 column tiles (a ragged last column and row tile); the
    # forward without a logits output is its own kernel instantiation (and the column tiles' scan
    # without bounds tests), so its argmax is checked against the oracle and against the forward
    # that writes the logits
    w, dl, OL = small
    log(f"small bf16 LM head without logits B={B} Nq={Nq}")
    L0, cap = 150, 320
    ctx = np.stack([synth.uniform_tokens(120 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(130 + b, Nq, SMALL.vocab) for b in range(B)])
    outs = []
    for logits in (False, True):
        cache = cad.DeviceCache(SMALL, B, cap)
        prefill(dl, cache, ctx, chunk=64)
        outs.append(run_forward(dl, cache, span, flags=cad.COMMIT_ALL, logits=logits))
        assert list(cache.len.cpu().numpy()) == [L0 + Nq] * B
    np.testing.assert_array_equal(outs[0]["argmax"], outs[1]["argmax"])
    np.testing.assert_array_equal(outs[0]["hidden"], outs[1]["hidden"])
    for b in range(B):
        oc = O.cache_from_tokens(OL, ctx[b], cap)
        ref = O.span_forward(OL, oc, span[b])
        rows = slice(b * Nq, (b + 1) * Nq)
        argmax_check(outs[0]["argmax"][rows], ref, outs[1]["logits"][rows], what=f"b={b} without logits")


@pytest.mark.parametrize("Nq", [1, 13, 40])
def test_small_bf16_copy_commit_last_row_matches_oracle(small, Nq):
    """Copy-commit mode (CAD_LOGITS_LAST): the LM head and argmax run for each sequence's last
    row only; the cache rows, hidden output and commit are those of the full forward."""
    w, dl, OL = small
    log(f"small bf16 copy-commit Nq={Nq}")
    B, L0, cap = 3, 150, 320
    ctx = np.stack([synth.uniform_tokens(50 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(70 + b, Nq, SMALL.vocab) for b in range(B)])
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx, chunk=64)
    t = torch.from_numpy(np.ascontiguousarray(span, dtype=np.int32)).cuda()
    am = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    hid = torch.zeros((B * Nq, SMALL.hidden), dtype=torch.int16, device="cuda")
    lg = torch.zeros((B, SMALL.vocab), dtype=torch.float32, device="cuda")
    cad.span_forward(dl, cache, t, Nq, flags=cad.COMMIT_ALL | cad.LOGITS_LAST, argmax_out=am, hidden_out=hid,
                     logits_out=lg)
    torch.cuda.synchronize()
    assert list(cache.len.cpu().numpy()) == [L0 + Nq] * B
    g_a, g_h, g_l = am.cpu().numpy(), to_f64(hid, "bf16"), lg.cpu().numpy().astype(np.float64)
    for b in range(B):
        oc = O.cache_from_tokens(OL, ctx[b], cap)
        ref = O.span_forward(OL, oc, span[b])
        rows = slice(b * Nq, (b + 1) * Nq)
        dh = np.abs(g_h[rows] - ref["hidden_out"])
        assert (dh <= hidden_tol(ref["hidden_out"], SMALL.ffn)).all(), f"b={b} hidden {dh.max()}"
        last = {k: ref[k][Nq - 1:Nq] for k in ("logits", "argmax", "top2_gap")}
        dl_ = np.max(np.abs(g_l[b:b + 1] - last["logits"]))
        assert dl_ <= LOGIT_TOL, f"b={b} last-row logits {dl_}"
        argmax_check(g_a[b:b + 1], last, g_l[b:b + 1], what=f"copy-commit b={b}")
        compare_cache(cache, b, oc, L0, L0 + Nq, "bf16", what=f"copy-commit rows b={b}")


def _allowed_sets(seed, rows, A, vocab, full_argmax):
    """Allowed-id sets of A slots per row: random ids, some padding (-1, vocab + 3), a duplicate,
    the unrestricted argmax in every third row, and one row that allows nothing."""
    rng = np.random.default_rng(seed)
    al = rng.integers(0, vocab, size=(rows, A)).astype(np.int32)
    for r in range(rows):
        k = r % 4
        if k == 1:
            al[r, -2:] = [-1, vocab + 3][-A:]
        elif k == 2 and A > 1:
            al[r, 1] = al[r, 0]
        if r % 3 == 0:
            al[r, r % A] = full_argmax[r]
    al[rows // 2] = -1
    return al


def _check_masked(g_a, g_v, al, ref_logits, vocab, what):
    best, vals, gap = O.masked_argmax(ref_logits, al, vocab)
    pad = ~np.isfinite(vals)
    assert (np.isneginf(g_v[pad])).all(), f"{what} padding slots must read -inf"
    d = np.where(pad, 0.0, np.abs(np.where(pad, 0.0, g_v) - np.where(pad, 0.0, vals)))
    e = d.max(axis=1)
    assert e.max() <= LOGIT_TOL, f"{what} allowed logits off by {e.max()}"
    none = best < 0
    assert (g_a[none] == -1).all(), f"{what} empty set must give -1"
    unique = ~none & (gap > np.maximum(NEAR_TIE, 2 * e))
    bad = np.nonzero(unique & (g_a != best))[0]
    assert bad.size == 0, f"{what} masked argmax differs at rows {bad[:10]}: {g_a[bad[:10]]} vs {best[bad[:10]]}"
    for r in np.nonzero(~none & ~unique)[0]:                  # near ties: a valid near-top allowed id
        ok = [int(a) for a in al[r] if 0 <= a < vocab]
        assert int(g_a[r]) in ok, f"{what} row {r} chose {g_a[r]} outside its set"
        assert ref_logits[r, ok].max() - ref_logits[r, g_a[r]] <= 2 * e[r] + 1e-12
    return int(unique.sum())


@pytest.mark.parametrize("Nq,A,commit,last", [(1, 12, True, False), (5, 16, True, False), (3, 1, False, False),
                                               (4, 11, True, True), (1, 2, False, True)])
def test_small_bf16_grammar_masked_argmax_matches_oracle(small, Nq, A, commit, last):
    """cad_span_forward_allowed: the argmax over each row's allowed ids equals the oracle's
    masked argmax on the oracle forward's logits (each sequence's last row only, with
    CAD_LOGITS_LAST); the cache rows, hidden output and commit are those of the full forward."""
    w, dl, OL = small
    log(f"small bf16 masked argmax Nq={Nq} A={A} commit={commit} last={last}")
    B, L0, cap = 3, 150, 320
    ctx = np.stack([synth.uniform_tokens(50 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(110 + b, Nq, SMALL.vocab) for b in range(B)])
    ocs = [O.cache_from_tokens(OL, ctx[b], cap) for b in range(B)]
    refs = [O.span_forward(OL, ocs[b], span[b]) for b in range(B)]       # appends the span rows to ocs[b]
    sel = slice(Nq - 1, Nq) if last else slice(0, Nq)
    ref_logits = np.concatenate([r["logits"][sel] for r in refs])
    ref_hidden = np.concatenate([r["hidden_out"] for r in refs])
    R = B if last else B * Nq
    al = _allowed_sets(7 * Nq + A, R, A, SMALL.vocab, np.concatenate([r["argmax"][sel] for r in refs]))
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx, chunk=64)
    t = torch.from_numpy(np.ascontiguousarray(span, dtype=np.int32)).cuda()
    ta = torch.from_numpy(al).cuda()
    am = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    lv = torch.zeros((R, A), dtype=torch.float32, device="cuda")
    hid = torch.zeros((B * Nq, SMALL.hidden), dtype=torch.int16, device="cuda")
    fl = (cad.COMMIT_ALL if commit else 0) | (cad.LOGITS_LAST if last else 0)
    cad.span_forward_allowed(dl, cache, t, Nq, ta, A, flags=fl, argmax_out=am, logits_out=lv, hidden_out=hid)
    torch.cuda.synchronize()
    assert list(cache.len.cpu().numpy()) == [L0 + Nq if commit else L0] * B
    dh = np.abs(to_f64(hid, "bf16") - ref_hidden)
    assert (dh <= hidden_tol(ref_hidden, SMALL.ffn)).all(), f"hidden {dh.max()}"
    n_unique = _check_masked(am.cpu().numpy(), lv.cpu().numpy().astype(np.float64), al, ref_logits, SMALL.vocab,
                             f"Nq={Nq} A={A}")
    assert n_unique >= R // 2
    for b in range(B):
        compare_cache(cache, b, ocs[b], L0, L0 + Nq, "bf16", what=f"masked rows b={b}")


def test_masked_argmax_over_the_top_ids_equals_the_plain_argmax(small):
    """A set holding the oracle's 16 largest logits of each row (in reverse order) gives the
    unrestricted argmax wherever that is unique."""
    w, dl, OL = small
    B, L0, cap, Nq, A = 2, 90, 128, 4, 16
    log("small bf16 masked argmax over the top-16 ids")
    ctx = np.stack([synth.uniform_tokens(30 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(40 + b, Nq, SMALL.vocab) for b in range(B)])
    refs = [O.span_forward(OL, O.cache_from_tokens(OL, ctx[b], cap), span[b]) for b in range(B)]
    lg = np.concatenate([r["logits"] for r in refs])
    top = np.ascontiguousarray(np.argsort(-lg, axis=1, kind="stable")[:, :A][:, ::-1], dtype=np.int32)
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx)
    t = torch.from_numpy(np.ascontiguousarray(span, dtype=np.int32)).cuda()
    am = torch.full((B * Nq,), -7, dtype=torch.int32, device="cuda")
    lv = torch.zeros((B * Nq, A), dtype=torch.float32, device="cuda")
    cad.span_forward_allowed(dl, cache, t, Nq, torch.from_numpy(top).cuda(), A, argmax_out=am, logits_out=lv)
    torch.cuda.synchronize()
    ga = am.cpu().numpy()
    _check_masked(ga, lv.cpu().numpy().astype(np.float64), top, lg, SMALL.vocab, "top-16")
    full = np.concatenate([r["argmax"] for r in refs])
    gap = np.concatenate([r["top2_gap"] for r in refs])
    assert (ga[gap > 2 * LOGIT_TOL] == full[gap > 2 * LOGIT_TOL]).all()


def test_tiny_fp32_masked_argmax_matches_oracle():
    """The masked decision on the fp32 layer (the fp32 instance of the allowed-ids kernel)."""
    wl = CONFIGS["tiny_f32"]
    w = synth.layer_weights(TINY, wl.seed)
    OL = oracle_layer(TINY, w)
    oc = O.cache_from_hidden(OL, synth.hidden_states(wl.seed, wl.cache_len, TINY.hidden), 160)
    span = synth.uniform_tokens(wl.seed, 8, TINY.vocab, stream=3)
    ref = O.span_forward(OL, oc.copy(), span)
    dl = cad.DeviceLayer(TINY, w)
    cache = cad.DeviceCache(TINY, 1, 160)
    upload_oracle_cache(cache, 0, oc, "f32")
    A = 9
    al = _allowed_sets(21, 8, A, TINY.vocab, ref["argmax"])
    am = torch.full((8,), -7, dtype=torch.int32, device="cuda")
    lv = torch.zeros((8, A), dtype=torch.float32, device="cuda")
    cad.span_forward_allowed(dl, cache, torch.from_numpy(span[None].astype(np.int32)).cuda(), 8,
                             torch.from_numpy(al).cuda(), A, flags=cad.COMMIT_ALL, argmax_out=am, logits_out=lv)
    torch.cuda.synchronize()
    assert int(cache.len[0]) == 128 + 8
    _check_masked(am.cpu().numpy(), lv.cpu().numpy().astype(np.float64), al, ref["logits"], TINY.vocab, "tiny fp32")


def test_sampled_forward_rejects_fp32_layers():
    wl = CONFIGS["tiny_f32"]
    dl = cad.DeviceLayer(TINY, synth.layer_weights(TINY, wl.seed))
    cache = cad.DeviceCache(TINY, 1, 32)
    t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    pred = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(cad.CadError) as e:
        cad.span_forward_sampled(dl, cache, t, 4, 1.0, 1, pred_out=pred)
    assert e.value.status == cad.CAD_EUNSUPPORTED


def test_copy_commit_mode_rejects_the_block_mask(small):
    w, dl, OL = small
    cache = cad.DeviceCache(SMALL, 1, 64)
    t = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    am = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(cad.CadError):
        cad.span_forward(dl, cache, t, 8, mode=cad.MASK_BLOCK, W=2, D=4, flags=cad.LOGITS_LAST, argmax_out=am)


@pytest.mark.parametrize("W, D", [(4, 8), (2, 9)])
def test_small_bf16_block_verify_matches_oracle(small, W, D):
    # (W, D) = (2, 9): 18 rows x 4 heads = 72 rows per GQA group, the two-key-phase attention tile
    w, dl, OL = small
    B, L0, cap = 2, 200, 260
    log(f"small bf16 block W={W} D={D}")
    ctx = np.stack([synth.uniform_tokens(80 + b, L0, SMALL.vocab) for b in range(B)])
    cand = np.stack([synth.uniform_tokens(90 + b, W * D, SMALL.vocab) for b in range(B)])
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx)
    g = run_forward(dl, cache, cand, mode=cad.MASK_BLOCK, W=W, D=D)
    assert list(cache.len.cpu().numpy()) == [L0] * B           # verify does not commit
    for b in range(B):
        oc = O.cache_from_tokens(OL, ctx[b], cap)
        ref = O.span_forward(OL, oc, cand[b], mode="block", W=W, D=D, commit=False)
        compare(g, ref, rows=slice(b * W * D, (b + 1) * W * D), what=f"block b={b}")


@pytest.mark.parametrize("mode, W, D, Nq", [("causal", 1, 0, 13), ("causal", 1, 0, 40), ("block", 2, 9, 18)])
def test_small_bf16_ragged_cache_lengths_match_oracle(small, mode, W, D, Nq):
    # one forward over sequences whose caches hold 0, 1, 63, 64, 65 and 200 positions: an empty
    # cache (the rows see only their own span) and lengths on both sides of a 64-key tile edge.
    # The caches are the oracle's own (exact in bf16), so both sides attend over the same keys.
    w, dl, OL = small
    lens = [0, 1, 63, 64, 65, 200]
    B, cap = len(lens), 320
    log(f"small bf16 ragged cache lengths {mode} Nq={Nq}")
    cache = cad.DeviceCache(SMALL, B, cap)
    ocs = []
    for b, L0 in enumerate(lens):
        oc = O.cache_from_tokens(OL, synth.uniform_tokens(140 + b, L0, SMALL.vocab), cap)
        upload_oracle_cache(cache, b, oc, "bf16")
        ocs.append(oc)
    span = np.stack([synth.uniform_tokens(150 + b, Nq, SMALL.vocab) for b in range(B)])
    commit = mode == "causal"
    g = run_forward(dl, cache, span, mode=cad.MASK_CAUSAL if commit else cad.MASK_BLOCK, W=W, D=max(D, 1),
                    flags=cad.COMMIT_ALL if commit else 0)
    assert list(cache.len.cpu().numpy()) == [L0 + (Nq if commit else 0) for L0 in lens]
    for b, L0 in enumerate(lens):
        ref = O.span_forward(OL, ocs[b], span[b], mode=mode, W=W, D=D, commit=commit)
        compare(g, ref, rows=slice(b * Nq, (b + 1) * Nq), what=f"{mode} b={b} len={L0}")
        if commit:
            compare_cache(cache, b, ocs[b], L0, L0 + Nq, "bf16", what=f"span rows b={b} len={L0}")


BF16_NAN = 0x7FC0   # a quiet NaN's bf16 bits (the device caches hold bf16 as int16)

# head_dim 64 with 4 query heads per KV head: spans of more than 16 positions take the 8-wave tile
SMALL_D64 = LayerShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1376, vocab=5003)


@pytest.fixture(scope="module")
def small_d64():
    w = synth.layer_weights(SMALL_D64, 78)
    return w, cad.DeviceLayer(SMALL_D64, w), oracle_layer(SMALL_D64, w)


@pytest.mark.parametrize("shape, Nq, W, D", [("d128", 8, 1, 0), ("d128", 17, 1, 0), ("d128", 40, 1, 0),
                                         ("d64", 40, 1, 0), ("d128", 18, 2, 9), ("d128", 32, 4, 8)])
def test_cache_slots_past_the_span_never_reach_the_output(small, small_d64, shape, Nq, W, D):
    # every cache slot at or past len + Nq holds NaN: the attention tiles read whole 64-key tiles
    # (K rows and V keys past the split's end), which must not reach any output.  Causal spans of
    # Nq = 8, 17 and 40 with head_dim 128 take the 4-, 10- and 8-wave tiles; head_dim 64 at
    # Nq = 40 the 8-wave tile; block verifies of 2 x 9 and 4 x 8 candidates the 10- and 8-wave
    # tiles.  Lengths on both sides of a tile edge, and 900 + Nq, whose splits hold several tiles
    # (the direct-copy tiles' loop and its ragged last tile).
    block = D > 0
    shp = SMALL if shape == "d128" else SMALL_D64
    w, dl, OL = small if shape == "d128" else small_d64
    lens = [0, 1, 63, 64, 65, 250, 900]
    B, cap = len(lens), 1024
    log(f"NaN past the span {shape} Nq={Nq} {'block' if block else 'causal'}")
    cache = cad.DeviceCache(shp, B, cap)
    ocs = []
    for b, L0 in enumerate(lens):
        oc = O.cache_from_tokens(OL, synth.uniform_tokens(190 + b, L0, shp.vocab), cap)
        upload_oracle_cache(cache, b, oc, "bf16")
        cache.k[b, :, L0 + Nq:] = BF16_NAN
        cache.v[b, :, :, L0 + Nq:] = BF16_NAN
        ocs.append(oc)
    span = np.stack([synth.uniform_tokens(200 + b, Nq, shp.vocab) for b in range(B)])
    if block:
        g = run_forward(dl, cache, span, mode=cad.MASK_BLOCK, W=W, D=D)
        assert list(cache.len.cpu().numpy()) == lens
    else:
        g = run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
        assert list(cache.len.cpu().numpy()) == [L0 + Nq for L0 in lens]
    for b, L0 in enumerate(lens):
        ref = (O.span_forward(OL, ocs[b], span[b], mode="block", W=W, D=D, commit=False) if block
               else O.span_forward(OL, ocs[b], span[b]))
        compare(g, ref, rows=slice(b * Nq, (b + 1) * Nq), what=f"NaN past span b={b} len={L0}")


@pytest.mark.parametrize("shape", ["d128", "d64"])
def test_small_bf16_multi_tile_splits_match_oracle(small, small_d64, shape):
    # 96-row spans over caches of 0..920 positions: three 128-row attention tiles per GQA group
    # and 7 key splits, so the longer sequences give each split two or three 64-key tiles (the
    # attention's cross-tile pipeline, its last tile ragged) while the short ones keep one-tile
    # splits; at head_dim 128 and 64 (one K and one V copy per wave and tile)
    shp = SMALL if shape == "d128" else SMALL_D64
    w, dl, OL = small if shape == "d128" else small_d64
    lens = [0, 200, 450, 700, 850, 920]
    B, Nq, cap = len(lens), 96, 1024
    log(f"small bf16 multi-tile attention splits {shape}")
    cache = cad.DeviceCache(shp, B, cap)
    ocs = []
    for b, L0 in enumerate(lens):
        oc = O.cache_from_tokens(OL, synth.uniform_tokens(170 + b, L0, shp.vocab), cap)
        upload_oracle_cache(cache, b, oc, "bf16")
        ocs.append(oc)
    span = np.stack([synth.uniform_tokens(180 + b, Nq, shp.vocab) for b in range(B)])
    g = run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
    assert list(cache.len.cpu().numpy()) == [L0 + Nq for L0 in lens]
    for b, L0 in enumerate(lens):
        ref = O.span_forward(OL, ocs[b], span[b])
        compare(g, ref, rows=slice(b * Nq, (b + 1) * Nq), what=f"multi-tile b={b} len={L0}")
        compare_cache(cache, b, ocs[b], L0, L0 + Nq, "bf16", what=f"span rows b={b} len={L0}")


def test_small_bf16_span_equals_decode_steps_on_gpu(small):
    w, dl, OL = small
    log("small bf16 span vs gpu decode steps")
    L0, N, cap = 90, 12, 128
    ctx = synth.uniform_tokens(33, L0, SMALL.vocab)[None]
    span = synth.uniform_tokens(34, N, SMALL.vocab)[None]
    c1, c2 = cad.DeviceCache(SMALL, 1, cap), cad.DeviceCache(SMALL, 1, cap)
    prefill(dl, c1, ctx)
    prefill(dl, c2, ctx)
    a = run_forward(dl, c1, span, flags=cad.COMMIT_ALL)
    steps = [run_forward(dl, c2, span[:, i:i + 1], flags=cad.COMMIT_ALL) for i in range(N)]
    b = {k: np.concatenate([s[k] for s in steps]) for k in ("argmax", "hidden", "logits")}
    ref = O.span_forward(OL, O.cache_from_tokens(OL, ctx[0], cap), span[0])
    compare(a, ref, what="span")
    compare(b, ref, what="decode steps")
    np.testing.assert_array_equal(c1.k.cpu().numpy(), c2.k.cpu().numpy())
    np.testing.assert_array_equal(c1.v.cpu().numpy(), c2.v.cpu().numpy())


def test_capacity_overflow_flags_and_skips(small):
    w, dl, OL = small
    log("capacity overflow")
    cache = cad.DeviceCache(SMALL, 2, 40)
    cache.len.copy_(torch.tensor([10, 35], dtype=torch.int32))
    span = synth.uniform_tokens(3, 2 * 8, SMALL.vocab).reshape(2, 8)
    g = run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
    assert list(cache.len.cpu().numpy()) == [18, 35]
    assert list(cache.err.cpu().numpy()) == [0, cad.CAD_ECAPACITY]
    assert (g["argmax"][8:] == -7).all()                       # nothing written for the flagged sequence


def test_sequence_filled_exactly_to_capacity(small):
    """len + Nq == cap is accepted and commits; the same span one slot later overflows."""
    w, dl, OL = small
    log("exact capacity")
    B, Nq, cap = 2, 12, 64
    ctx = np.stack([synth.uniform_tokens(150 + b, cap - Nq, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(160 + b, Nq, SMALL.vocab) for b in range(B)])
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx, chunk=64)
    g = run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
    assert list(cache.len.cpu().numpy()) == [cap] * B and not cache.err.any()
    for b in range(B):
        oc = O.cache_from_tokens(OL, ctx[b], cap)
        ref = O.span_forward(OL, oc, span[b])
        compare(g, ref, rows=slice(b * Nq, (b + 1) * Nq), what=f"full cache b={b}")
        compare_cache(cache, b, oc, cap - Nq, cap, "bf16", what=f"last rows b={b}")
    cache.len.fill_(cap - Nq + 1)
    run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
    assert list(cache.err.cpu().numpy()) == [cad.CAD_ECAPACITY] * B
    assert list(cache.len.cpu().numpy()) == [cap - Nq + 1] * B


def test_argument_errors_are_reported_before_any_work(small):
    """Host-visible argument errors return a negative status and enqueue nothing."""
    w, dl, OL = small
    log("argument errors")
    cache = cad.DeviceCache(SMALL, 2, 64)
    t = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    am = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    ws = cad.alloc_workspace(cad.span_forward_workspace(dl, 2, 8, cad.MASK_CAUSAL, 1, 1, 64, 0))

    def status(fn):
        try:
            fn()
        except cad.CadError as e:
            return e.status
        return cad.CAD_OK

    assert status(lambda: cad.span_forward(dl, cache, t, 0, argmax_out=am, workspace=ws)) == cad.CAD_EINVAL
    assert status(lambda: cad.span_forward(dl, cache, t, 8, mode=cad.MASK_BLOCK, W=3, D=4, argmax_out=am,
                                           workspace=ws)) == cad.CAD_EINVAL          # W*D != Nq
    assert status(lambda: cad.span_forward(dl, cache, t, 8, flags=8, argmax_out=am, workspace=ws)) == cad.CAD_EINVAL
    assert status(lambda: cad.span_forward(dl, cache, t, 8, workspace=ws)) == cad.CAD_EINVAL   # no argmax_out
    small_ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    assert status(lambda: cad.span_forward(dl, cache, t, 8, argmax_out=am, workspace=small_ws)) == cad.CAD_EWORKSPACE
    odd = cad.DeviceCache(SMALL, 2, 66)                                               # cap not a multiple of 4
    assert status(lambda: cad.span_forward(dl, odd, t, 8, argmax_out=am)) == cad.CAD_EUNSUPPORTED
    d = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    dlen = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    ctx = torch.zeros((2, 32), dtype=torch.int32, device="cuda")
    clen = torch.zeros(2, dtype=torch.int32, device="cuda")
    assert status(lambda: cad.ngram_lookup(ctx, clen, 0, 1, 8, 0, d, dlen)) == cad.CAD_EINVAL           # n = 0
    assert status(lambda: cad.ngram_lookup(ctx, clen, 3, 9, 8, 0, d, dlen)) == cad.CAD_EUNSUPPORTED     # W > 8
    torch.cuda.synchronize()
    assert not cache.len.any() and not cache.err.any()                                # nothing ran


def test_forward_is_deterministic(small):
    w, dl, OL = small
    log("determinism")
    ctx = synth.uniform_tokens(41, 120, SMALL.vocab)[None]
    span = synth.uniform_tokens(42, 37, SMALL.vocab)[None]
    outs = []
    for _ in range(2):
        c = cad.DeviceCache(SMALL, 1, 200)
        prefill(dl, c, ctx)
        outs.append(run_forward(dl, c, span))
    for k in ("argmax", "hidden", "logits"):
        np.testing.assert_array_equal(outs[0][k], outs[1][k])


def test_forward_replays_from_a_hip_graph(small):
    # bench.py replays forwards from HIP graphs: every replay must reproduce the eager result,
    # with the program's own eager work and synchronisations between replays
    w, dl, OL = small
    log("graph replay")
    L0, N, cap = 120, 21, 200
    ctx = synth.uniform_tokens(43, L0, SMALL.vocab)[None]
    span = torch.from_numpy(synth.uniform_tokens(44, N, SMALL.vocab)[None].astype(np.int32)).cuda()
    cache = cad.DeviceCache(SMALL, 1, cap)
    prefill(dl, cache, ctx)
    am = torch.zeros((1, N), dtype=torch.int32, device="cuda")
    hid = torch.zeros((N, SMALL.hidden), dtype=torch.int16, device="cuda")
    lg = torch.zeros((N, SMALL.vocab), dtype=torch.float32, device="cuda")
    ws = cad.alloc_workspace(cad.span_forward_workspace(dl, 1, N, cad.MASK_CAUSAL, 1, 1, cap, cad.COMMIT_ALL))

    def fwd(stream):
        cache.len.fill_(L0)
        cad.span_forward(dl, cache, span, N, flags=cad.COMMIT_ALL, argmax_out=am, hidden_out=hid, logits_out=lg,
                         workspace=ws, stream=stream)

    fwd(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = [t.clone() for t in (am, hid, lg, cache.k, cache.v)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fwd(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (am, hid, lg):
            t.zero_()
        cache.len.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((am, hid, lg, cache.k, cache.v), eager):
            assert torch.equal(a, b), f"replay {rep}"
        assert int(cache.len[0]) == L0 + N


# ------------------------------------------------------------------------- top-2 gap, bad ids, skipped accepts
@pytest.mark.parametrize("B,Nq,last", [(1, 8, False), (3, 13, False), (1, 40, False), (1, 100, False),
                                       (2, 150, False), (3, 13, True)])
def test_top2_gap_matches_oracle(small, B, Nq, last):
    """The top-2 gap output against the oracle's (largest minus second-largest logit).  Each logit
    is within the row's measured error e of the oracle's, so the two largest are too and the gap
    is within 2e; the rows cover the weight-streaming LM head (<= 32 rows), the balanced-range
    tiled one (33-128) and the column-tile one (300 rows)."""
    w, dl, OL = small
    log(f"top2 gap B={B} Nq={Nq} last={last}")
    L0, cap = 60, (60 + Nq + 4 + 3) // 4 * 4
    ctx = np.stack([synth.uniform_tokens(700 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(710 + b, Nq, SMALL.vocab) for b in range(B)])
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx, chunk=64)
    R = B if last else B * Nq
    t = torch.from_numpy(span.astype(np.int32)).cuda()
    am = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    gap = torch.full((R,), -7.0, dtype=torch.float32, device="cuda")
    lg = torch.zeros((R, SMALL.vocab), dtype=torch.float32, device="cuda")
    flags = cad.COMMIT_ALL | (cad.LOGITS_LAST if last else 0)
    cad.span_forward(dl, cache, t, Nq, flags=flags, argmax_out=am, logits_out=lg, top2_gap=gap)
    # the same forward without logits (the hot instantiations) gives the same gap bits
    cache.len.fill_(L0)
    am2 = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    gap2 = torch.full((R,), -7.0, dtype=torch.float32, device="cuda")
    cad.span_forward(dl, cache, t, Nq, flags=flags, argmax_out=am2, top2_gap=gap2)
    torch.cuda.synchronize()
    g_gap, g_l = gap.cpu().numpy().astype(np.float64), lg.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(gap2.cpu().numpy(), gap.cpu().numpy())
    np.testing.assert_array_equal(am2.cpu().numpy(), am.cpu().numpy())
    # the gap is exactly the one the GPU's own logits give (an fp32 difference)
    srt = np.sort(lg.cpu().numpy(), axis=1)
    np.testing.assert_array_equal(gap.cpu().numpy(), srt[:, -1] - srt[:, -2])
    for b in range(B):
        ref = O.span_forward(OL, O.cache_from_tokens(OL, ctx[b], cap), span[b])
        rows = slice(b, b + 1) if last else slice(b * Nq, (b + 1) * Nq)
        ref_gap = ref["top2_gap"][Nq - 1:Nq] if last else ref["top2_gap"]
        ref_l = ref["logits"][Nq - 1:Nq] if last else ref["logits"]
        e = np.max(np.abs(g_l[rows] - ref_l), axis=1)
        assert (np.abs(g_gap[rows] - ref_gap) <= 2 * e + 1e-12).all()


def test_tiny_fp32_top2_gap_matches_oracle():
    wl = CONFIGS["tiny_f32"]
    w = synth.layer_weights(TINY, wl.seed)
    OL, dl = oracle_layer(TINY, w), cad.DeviceLayer(TINY, w)
    log("tiny fp32 top2 gap")
    ctx = synth.uniform_tokens(720, 40, TINY.vocab)
    span = synth.uniform_tokens(721, 8, TINY.vocab)
    cache = cad.DeviceCache(TINY, 1, 64)
    prefill(dl, cache, ctx[None], chunk=64)
    t = torch.from_numpy(span[None].astype(np.int32)).cuda()
    am = torch.zeros(8, dtype=torch.int32, device="cuda")
    gap = torch.zeros(8, dtype=torch.float32, device="cuda")
    lg = torch.zeros((8, TINY.vocab), dtype=torch.float32, device="cuda")
    cad.span_forward(dl, cache, t, 8, argmax_out=am, logits_out=lg, top2_gap=gap)
    torch.cuda.synchronize()
    ref = O.span_forward(OL, O.cache_from_tokens(OL, ctx, 64), span)
    e = np.max(np.abs(lg.cpu().numpy() - ref["logits"]), axis=1)
    assert (np.abs(gap.cpu().numpy() - ref["top2_gap"]) <= 2 * e + 1e-9).all()


def test_out_of_range_token_ids_flag_only_their_sequence(small):
    """A sequence holding an id outside [0, vocab) is flagged CAD_EINVAL and left untouched (no
    cache rows, no outputs, no commit); the other sequences of the batch are computed as usual."""
    w, dl, OL = small
    log("out-of-range token ids")
    B, Nq, L0, cap = 3, 12, 50, 72
    ctx = np.stack([synth.uniform_tokens(730 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(740 + b, Nq, SMALL.vocab) for b in range(B)]).astype(np.int64)
    span[1, 5] = SMALL.vocab
    span[2, 0] = -1
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl, cache, ctx, chunk=64)
    k_before = cache.k.clone()
    g = run_forward(dl, cache, span, flags=cad.COMMIT_ALL)
    assert list(cache.len.cpu().numpy()) == [L0 + Nq, L0, L0]
    assert list(cache.err.cpu().numpy()) == [0, cad.CAD_EINVAL, cad.CAD_EINVAL]
    assert (g["argmax"][Nq:] == -7).all()
    assert torch.equal(cache.k[1:], k_before[1:])
    ref = O.span_forward(OL, O.cache_from_tokens(OL, ctx[0], cap), span[0])
    compare(g, ref, rows=slice(0, Nq), what="valid sequence beside flagged ones")


def test_accept_scan_skipped_sequences_report_nothing():
    """Sequences the scan skips (error flag already set; history overflow without a cache) get
    accepted = 0, n_emitted = 0, a zero emitted row and unchanged lengths."""
    log("accept skipped sequences")
    B, D = 4, 6
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    rows = np.arange(B * (1 + D)).reshape(B, 1 + D) % 7
    pred = rows[:, 1:].copy()
    pred = np.concatenate([pred, np.full((B, 1), 3)], axis=1)          # every draft agrees: a = D
    dl = np.full((B, 1), D)
    cache = cad.DeviceCache(SMALL, B, 64)
    cache.len.copy_(torch.tensor([10, 10, 10, 10], dtype=torch.int32))
    cache.err.copy_(torch.tensor([0, cad.CAD_ECAPACITY, 0, 0], dtype=torch.int32))
    acc, bw, ne = (torch.full((B,), -1, dtype=torch.int32, device="cuda") for _ in range(3))
    em = torch.full((B, D + 1), -1, dtype=torch.int32, device="cuda")
    ctx = torch.zeros((B, 32), dtype=torch.int32, device="cuda")
    clen = T([0, 0, 30, 0])                                            # sequence 2's history is full
    cad.accept_scan(T(rows), 1, T(dl), T(pred), None, B, 1, D, cad.MASK_CAUSAL, acc, bw, em, ne,
                    ctx=ctx, ctx_len=clen, ctx_cap=32, cache=cache)
    torch.cuda.synchronize()
    assert list(acc.cpu().numpy()) == [D, 0, 0, D]
    assert list(ne.cpu().numpy()) == [D + 1, 0, 0, D + 1]
    assert list(bw.cpu().numpy()) == [0, 0, 0, 0]
    assert not em[1:3].any()
    assert list(cache.len.cpu().numpy()) == [10 + D + 1, 10, 10, 10 + D + 1]
    assert list(clen.cpu().numpy()) == [D + 1, 0, 30, D + 1]
    assert list(cache.err.cpu().numpy()) == [0, cad.CAD_ECAPACITY, cad.CAD_ECAPACITY, 0]
    # without a cache a history overflow is still visible: n_emitted = 0
    clen2 = T([0, 30, 0, 0])
    ne.fill_(-1)
    cad.accept_scan(T(rows), 1, T(dl), T(pred), None, B, 1, D, cad.MASK_CAUSAL, acc, None, em, ne,
                    ctx=ctx, ctx_len=clen2, ctx_cap=32)
    torch.cuda.synchronize()
    assert list(ne.cpu().numpy()) == [D + 1, 0, D + 1, D + 1]
    assert list(clen2.cpu().numpy()) == [D + 1, 30, D + 1, D + 1]
