"""GPU parity of the sampled span forward (stochastic verification) against the oracle.

The draws depend on the logits through Gumbel-perturbed maxima and the acceptance test
u < p(d); the GPU's logits differ from the oracle's by up to a measured row error e (fp32 vs
fp64 accumulation), so a decision must match bit for bit where the oracle takes it with a margin
the error cannot cross: a perturbed top-2 gap above 2e/T, or |u - p(d)| / p(d) above
exp(2e/T) - 1.  Elsewhere the GPU's token must be a valid near-top choice."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from spec_verify_cad_amd import cad, synth
from spec_verify_cad_amd.configs import SMALL

from gpu_util import log, prefill

pytestmark = pytest.mark.gpu

T32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.fixture(scope="module")
def small():
    from helpers import oracle_layer
    w = synth.layer_weights(SMALL, 77)
    return w, cad.DeviceLayer(SMALL, w), oracle_layer(SMALL, w)


def _greedy_chain(OL, ctx, cap, first, k):
    c = O.cache_from_tokens(OL, ctx, cap)
    out, t = [], first
    for _ in range(k):
        t = int(O.decode_one(OL, c, t)["argmax"][0])
        out.append(t)
    return out


def _check_rows(g_pred, g_logits, ref_logits, toks, dl, T, seed, b, base, what):
    pred, y, z, pd, u = O.sampled_predictions(ref_logits, toks, dl, T, seed, b, base)
    y_gap, z_gap, acc_m = O.sampled_margins(ref_logits, toks, dl, T, seed, b, base)
    e = np.max(np.abs(g_logits - ref_logits), axis=1)
    firm = np.zeros(len(pred), dtype=bool)
    for i in range(len(pred)):
        if i < dl:
            acc_firm = acc_m[i] > math.expm1(2 * e[i] / T) + 1e-6
            kept = u[i] < pd[i]
            firm[i] = acc_firm and (kept or z_gap[i] > 2 * e[i] / T + 1e-6)
        else:
            firm[i] = y_gap[i] > 2 * e[i] / T + 1e-6
        if firm[i]:
            assert g_pred[i] == pred[i], f"{what} row {i}: gpu {g_pred[i]} oracle {pred[i]} (draft row {i < dl})"
        else:
            assert 0 <= g_pred[i] < ref_logits.shape[1]
    return pred, firm


@pytest.mark.parametrize("T", [0.05, 1.3])
def test_small_sampled_verify_matches_oracle(small, T):
    """Random weights give a flat target (logits of a few tenths), so a greedy draft is kept
    often only at a small temperature; at T = 1.3 the rows are nearly uniform draws."""
    w, dl_, OL = small
    B, L0, cap, k = 3, 120, 200, 10
    Nq = k + 1
    seed = 0x1234_5678_9ABC + int(T * 10)
    log(f"sampled verify T={T}")
    ctx = np.stack([synth.uniform_tokens(400 + b, L0, SMALL.vocab) for b in range(B)])
    g = [int(x) for x in synth.uniform_tokens(410, B, SMALL.vocab)]
    # sequence 0 drafts the greedy continuation (mostly kept), 1 random tokens (mostly replaced),
    # 2 drafts nothing (plain draws)
    drafts = [_greedy_chain(OL, ctx[0], cap, g[0], k), list(synth.uniform_tokens(411, k, SMALL.vocab)), [0] * k]
    dls = [k, 6, 0]
    toks = np.array([[g[b]] + drafts[b] for b in range(B)], dtype=np.int32)
    cache = cad.DeviceCache(SMALL, B, cap)
    prefill(dl_, cache, ctx, chunk=64)
    pred = torch.full((B * Nq,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros((B * Nq, SMALL.vocab), dtype=torch.float32, device="cuda")
    cad.span_forward_sampled(dl_, cache, T32(toks), Nq, T, seed, draft_len=T32(dls), pred_out=pred, logits_out=lg)
    torch.cuda.synchronize()
    assert list(cache.len.cpu().numpy()) == [L0] * B                  # a verify forward does not commit
    g_pred, g_l = pred.cpu().numpy(), lg.cpu().numpy().astype(np.float64)
    kept_total = 0
    for b in range(B):
        ref = O.span_forward(OL, O.cache_from_tokens(OL, ctx[b], cap), toks[b])
        rows = slice(b * Nq, (b + 1) * Nq)
        opred, firm = _check_rows(g_pred[rows], g_l[rows], ref["logits"], toks[b], dls[b], T, seed, b, L0, f"b={b}")
        kept_total += sum(1 for i in range(dls[b]) if opred[i] == toks[b, i + 1])
        log(f"b={b}: {int(firm.sum())}/{Nq} rows firm, kept drafts {[int(opred[i] == toks[b, i + 1]) for i in range(dls[b])]}")
        # the accept scan on the GPU predictions gives the oracle's stochastic result
        a_ref, em_ref = O.accept_causal(toks[b, 1:], dls[b], opred)
        if firm[:a_ref + 1].all():
            acc, bw, ne = (torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(3))
            em = torch.zeros((1, Nq), dtype=torch.int32, device="cuda")
            cad.accept_scan(T32(toks[b:b + 1]), 1, T32([dls[b]]), T32(g_pred[rows][None]), None, 1, 1, k,
                            cad.MASK_CAUSAL, acc, bw, em, ne)
            torch.cuda.synchronize()
            assert acc.item() == a_ref and list(em[0, :ne.item()].cpu().numpy()) == em_ref
    if T < 0.5:
        assert kept_total >= 1


def test_draws_do_not_depend_on_the_launch_shape(small):
    """A row's plain draw is keyed by (seed, sequence, position): the last row of a 9-row sampled
    forward, the same row alone in copy-commit mode, and a one-row forward at that position agree."""
    w, dl_, OL = small
    B, L0, cap, Nq, T, seed = 2, 60, 100, 9, 1.0, 99
    ctx = np.stack([synth.uniform_tokens(420 + b, L0, SMALL.vocab) for b in range(B)])
    span = np.stack([synth.uniform_tokens(430 + b, Nq, SMALL.vocab) for b in range(B)])
    c1, c2, c3 = (cad.DeviceCache(SMALL, B, cap) for _ in range(3))
    for c in (c1, c2, c3):
        prefill(dl_, c, ctx)
    full = torch.zeros(B * Nq, dtype=torch.int32, device="cuda")
    last = torch.zeros(B, dtype=torch.int32, device="cuda")
    one = torch.zeros(B, dtype=torch.int32, device="cuda")
    cad.span_forward_sampled(dl_, c1, T32(span), Nq, T, seed, pred_out=full, flags=cad.COMMIT_ALL)
    cad.span_forward_sampled(dl_, c2, T32(span), Nq, T, seed, pred_out=last, flags=cad.COMMIT_ALL | cad.LOGITS_LAST)
    cad.span_forward(dl_, c3, T32(span[:, :Nq - 1]), Nq - 1, flags=cad.COMMIT_ALL | cad.KV_ONLY)
    cad.span_forward_sampled(dl_, c3, T32(span[:, Nq - 1:]), 1, T, seed, pred_out=one, flags=cad.COMMIT_ALL)
    torch.cuda.synchronize()
    f = full.cpu().numpy().reshape(B, Nq)[:, -1]
    assert list(f) == list(last.cpu().numpy()) == list(one.cpu().numpy())
    assert list(c1.len.cpu().numpy()) == list(c2.len.cpu().numpy()) == list(c3.len.cpu().numpy()) == [L0 + Nq] * B
    # and they are the oracle's draws where the oracle is firm
    for b in range(B):
        ref = O.span_forward(OL, O.cache_from_tokens(OL, ctx[b], cap), span[b])
        y_gap, _, _ = O.sampled_margins(ref["logits"][-1:], span[b, -1:], 0, T, seed, b, L0 + Nq - 1)
        y = O.sampled_predictions(ref["logits"][-1:], span[b, -1:], 0, T, seed, b, L0 + Nq - 1)[1]
        if y_gap[0] > 0.05:
            assert f[b] == y[0]


def test_sampled_argument_errors(small):
    w, dl_, OL = small
    cache = cad.DeviceCache(SMALL, 1, 64)
    t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    pred = torch.zeros(4, dtype=torch.int32, device="cuda")
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(cad.CadError):
            cad.span_forward_sampled(dl_, cache, t, 4, T, 1, pred_out=pred)
    with pytest.raises(cad.CadError):
        cad.span_forward_sampled(dl_, cache, t, 4, 1.0, 1, pred_out=pred, flags=cad.KV_ONLY)
    torch.cuda.synchronize()
    assert int(cache.len[0]) == 0
