"""Helpers shared by the GPU parity tests: device layers/caches from seeded inputs,
KV-only prefill through the library, and oracle comparisons (tolerances of the contract:
bit-exact integers and argmax away from near-ties, max-abs 2e-2 on bf16 hidden outputs,
1e-2 on fp32 logits)."""
import numpy as np
import torch

import oracle as O
from spec_verify_cad_amd import cad, synth

from helpers import oracle_layer

HIDDEN_TOL = 2e-2
LOGIT_TOL = 1e-2
NEAR_TIE = 1e-3


def log(msg):
    print(f"[gpu] {msg}", flush=True)


def to_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.detach().cpu()
    if dtype == "bf16":
        return O.decode_bf16_bits(a.numpy().view(np.uint16))
    return a.numpy().astype(np.float64)


def prefill(layer: cad.DeviceLayer, cache: cad.DeviceCache, tokens: np.ndarray, chunk: int = 2048):
    """Append a [B, L] token prefix to the cache with KV-only forwards."""
    B, Lp = tokens.shape
    for s in range(0, Lp, chunk):
        t = torch.from_numpy(np.ascontiguousarray(tokens[:, s:s + chunk], dtype=np.int32)).cuda()
        cad.span_forward(layer, cache, t, t.shape[1], flags=cad.KV_ONLY | cad.COMMIT_ALL)


def upload_oracle_cache(cache: cad.DeviceCache, b: int, oc: O.Cache, dtype: str):
    """Copy an oracle cache into sequence b of a device cache (an oracle-made input)."""
    n = oc.length
    for name, src in (("k", oc.K), ("v", oc.V)):
        dst = getattr(cache, name)
        if dtype == "bf16":
            bits = synth.f32_to_bf16_bits(src[:, :n].astype(np.float32))   # exact: values are bf16
            dst[b, :, :n] = torch.from_numpy(bits.view(np.int16)).cuda()
        else:
            dst[b, :, :n] = torch.from_numpy(src[:, :n].astype(np.float32)).cuda()
    cache.len[b] = n


def run_forward(layer, cache, tokens: np.ndarray, mode=cad.MASK_CAUSAL, W=1, D=1, flags=0, logits=True):
    B, Nq = tokens.shape
    s = layer.shape
    t = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).cuda()
    am = torch.full((B, Nq), -7, dtype=torch.int32, device="cuda")
    hdt = torch.int16 if s.dtype == "bf16" else torch.float32
    hid = torch.zeros((B * Nq, s.hidden), dtype=hdt, device="cuda")
    lg = torch.zeros((B * Nq, s.vocab), dtype=torch.float32, device="cuda") if logits else None
    cad.span_forward(layer, cache, t, Nq, mode, W, D, flags, am, hid, lg)
    torch.cuda.synchronize()
    return {"argmax": am.cpu().numpy().reshape(-1), "hidden": to_f64(hid, s.dtype),
            "logits": None if lg is None else lg.cpu().numpy().astype(np.float64)}


def compare(gpu: dict, ref: dict, rows=None, what=""):
    """GPU forward outputs against an oracle forward (rows: subset of GPU rows to use)."""
    g_h = gpu["hidden"] if rows is None else gpu["hidden"][rows]
    g_a = gpu["argmax"] if rows is None else gpu["argmax"][rows]
    dh = np.max(np.abs(g_h - ref["hidden_out"]))
    assert dh <= HIDDEN_TOL, f"{what} hidden max-abs {dh}"
    if gpu["logits"] is not None:
        g_l = gpu["logits"] if rows is None else gpu["logits"][rows]
        dl = np.max(np.abs(g_l - ref["logits"]))
        assert dl <= LOGIT_TOL, f"{what} logits max-abs {dl} (hidden {dh})"
    log(f"{what} hidden max-abs {dh:.3e}" + (f" logits max-abs {dl:.3e}" if gpu["logits"] is not None else ""))
    sure = ref["top2_gap"] >= NEAR_TIE
    bad = np.nonzero((g_a != ref["argmax"]) & sure)[0]
    assert bad.size == 0, f"{what} argmax differs at rows {bad[:10]}: gpu {g_a[bad[:10]]} oracle {ref['argmax'][bad[:10]]}"
    return dh


def compare_cache(cache: cad.DeviceCache, b: int, oc: O.Cache, lo: int, hi: int, dtype: str, what=""):
    """Cache rows [lo, hi) of sequence b against the oracle's.  A stored k/v element is a
    rounded dot product of a rounded normed input; where the two sides round that input
    differently (fp32 vs fp64 accumulation just below a rounding boundary) a small element can
    move by several of its own ulps, so the bound is absolute (the hidden-output tolerance for
    bf16, 1e-5 for fp32) and almost every element must be bit-identical."""
    tol = HIDDEN_TOL if dtype == "bf16" else 1e-5
    for name, ref in (("k", oc.K), ("v", oc.V)):
        got = to_f64(getattr(cache, name)[b, :, lo:hi], dtype)
        want = ref[:, lo:hi]
        diff = np.abs(got - want)
        assert np.max(diff) <= tol, f"{what} {name} max-abs {np.max(diff)}"
        frac = np.mean(diff > 0)
        assert frac < 0.01, f"{what} {name} differing fraction {frac}"
