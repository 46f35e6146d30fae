"""Independent pin of the oracle's whole layer: the same pre-norm decoder layer composed from
torch fp64 primitives (F.rms_norm, F.silu, F.scaled_dot_product_attention with grouped-query
heads, complex-number RoPE, plain matmuls), sharing no code with `oracle.cad_oracle`.

Copy-as-Decode §2.4 makes the splice an ordinary forward over the N new tokens, so every part
of the layer enters the result: the O projection and residual, the MLP's input norm, the SwiGLU
product, the down projection and residual, the final norm and the LM head.  The span-equals-
decode pins cannot see an error both of the oracle's paths share; this composition can.

Rounding at the contract points R1-R8 is done here with an arithmetic round-half-to-even
(scale by the bf16 ulp of the value, torch.round, scale back), not with torch's bf16 cast: that
cast goes fp64 -> fp32 -> bf16 and double-rounds about one value in 2^16.

Comparison: hidden outputs (bf16 values) and argmax ids bit-exact; logits (fp32) bit-exact in
at least 99.99 % of the elements and never more than one fp32 ulp apart (the two sides sum the
fp64 dot products in different orders, so an fp32 rounding can fall differently where the fp64
sum lies within a few fp64 ulps of an fp32 midpoint)."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import oracle.cad_oracle as OC
from spec_verify_cad_amd import synth
from spec_verify_cad_amd.configs import SMALL
from spec_verify_cad_amd.synth import LayerShape

from helpers import oracle_layer

MINI = LayerShape(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=192, vocab=211)

f64 = torch.float64


def rne_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round fp64 values to bf16 precision (8 significant bits), ties to even, in fp64."""
    m, e = torch.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    ulp_exp = (e - 8).to(f64)                   # bf16 keeps 8 bits: ulp = 2^(e - 8)
    q = torch.ldexp(x, -ulp_exp)                # exact power-of-two scaling
    return torch.where(x == 0, x, torch.ldexp(torch.round(q), ulp_exp))


def rnd_f32(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float32).to(f64)


class TorchLayer:
    """The layer's weights as torch fp64 tensors, split from the library's packed layout."""

    def __init__(self, shape: LayerShape, w: dict):
        dec = lambda a: torch.from_numpy(
            (a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a).to(f64)
        self.s = shape
        qd, kd = shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
        qkv, gu = dec(w["w_qkv"]), dec(w["w_gate_up"])
        self.embed, self.wo, self.wd, self.wlm = dec(w["embed"]), dec(w["w_o"]), dec(w["w_down"]), dec(w["w_lm"])
        self.wq, self.wk, self.wv = qkv[:qd], qkv[qd:qd + kd], qkv[qd + kd:]
        self.wg, self.wu = gu[:shape.ffn], gu[shape.ffn:]

    def norm(self, x):
        return F.rms_norm(x, (x.shape[-1],), eps=self.s.rms_eps)

    def rope(self, x, pos):
        """Half-split rotary embedding as a complex rotation: (a, b) -> (a + ib) * e^(i*p*theta)."""
        d = x.shape[-1]
        theta = self.s.rope_base ** (-torch.arange(0, d // 2, dtype=f64) * 2.0 / d)
        rot = torch.polar(torch.ones(len(pos), d // 2, dtype=f64), pos.to(f64)[:, None] * theta[None, :])
        z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    def kv(self, u, pos):
        s = self.s
        k = self.rope((u @ self.wk.T).view(-1, s.n_kv_heads, s.head_dim), pos)
        v = (u @ self.wv.T).view(-1, s.n_kv_heads, s.head_dim)
        return rne_bf16(k), rne_bf16(v)                                  # R3

    def forward(self, prefix, span, mode="causal", W=1, D=0):
        """Prefill the prefix's K/V, then the span forward (append-then-attend) through the
        layer, final norm and LM head.  Returns hidden_out, logits, argmax."""
        s = self.s
        prefix, span = torch.as_tensor(prefix), torch.as_tensor(span)
        Lp, n = len(prefix), len(span)
        kp, vp = self.kv(rne_bf16(self.norm(self.embed[prefix])), torch.arange(Lp))
        x = self.embed[span]
        u = rne_bf16(self.norm(x))                                       # R1
        if mode == "causal":
            pos = Lp + torch.arange(n)
            allow = torch.ones(n, n, dtype=torch.bool).tril()
        else:
            j = torch.arange(n) % D
            cand = torch.arange(n) // D
            pos = Lp + j
            allow = (cand[:, None] == cand[None, :]) & (j[None, :] <= j[:, None])
        q = rne_bf16(self.rope((u @ self.wq.T).view(n, s.n_q_heads, s.head_dim), pos))   # R2
        ks, vs = self.kv(u, pos)
        K, V = torch.cat([kp, ks]), torch.cat([vp, vs])                  # [Lp+n, Hkv, d]
        mask = torch.cat([torch.ones(n, Lp, dtype=torch.bool), allow], dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), K.transpose(0, 1), V.transpose(0, 1),
                                           attn_mask=mask, enable_gqa=True)
        o = rne_bf16(o.transpose(0, 1).reshape(n, -1))                   # R4
        h1 = rnd_f32(x + o @ self.wo.T)
        u2 = rne_bf16(self.norm(h1))                                     # R5
        act = rne_bf16(F.silu(u2 @ self.wg.T) * (u2 @ self.wu.T))        # R6
        h2 = rnd_f32(h1 + act @ self.wd.T)
        u3 = rne_bf16(self.norm(h2))                                     # R8
        logits = rnd_f32(u3 @ self.wlm.T)
        return {"hidden_out": rne_bf16(h2).numpy(), "logits": logits.numpy(),   # R7
                "argmax": torch.argmax(logits, dim=-1).numpy()}


def _case(shape, seed, Lp, n, mode, W=1, D=0):
    w = synth.layer_weights(shape, seed)
    prefix = synth.uniform_tokens(seed, Lp, shape.vocab)
    span = synth.uniform_tokens(seed, n, shape.vocab, stream=1)
    L = oracle_layer(shape, w)
    cache = O.cache_from_tokens(L, prefix, Lp + n)
    ref = O.span_forward(L, cache, span, mode, W, D)
    got = TorchLayer(shape, w).forward(prefix, span, mode, W, D)
    return ref, got


def _agree(ref, got):
    """The pin's bar: hidden and argmax bit-exact, logits exact up to the summation-order
    allowance stated in the module docstring.  Returns a description of the first failure."""
    if not np.array_equal(ref["hidden_out"], got["hidden_out"]):
        return f"hidden_out differs in {int(np.sum(ref['hidden_out'] != got['hidden_out']))} elements"
    if not np.array_equal(ref["argmax"], got["argmax"]):
        return "argmax differs"
    a, b = ref["logits"].astype(np.float32), got["logits"].astype(np.float32)
    ulps = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
    if ulps.max() > 1 or np.mean(ulps == 0) < 0.9999:
        return f"logits differ (max {ulps.max()} ulp, exact {np.mean(ulps == 0):.6f})"
    return None


CASES = [
    (MINI, 21, 37, 13, "causal", 1, 0),
    (MINI, 22, 50, 12, "block", 3, 4),
    (SMALL, 23, 90, 40, "causal", 1, 0),
    (SMALL, 24, 70, 32, "block", 4, 8),
]


@pytest.mark.parametrize("shape,seed,Lp,n,mode,W,D", CASES)
def test_torch_composed_layer_equals_oracle(shape, seed, Lp, n, mode, W, D):
    ref, got = _case(shape, seed, Lp, n, mode, W, D)
    err = _agree(ref, got)
    assert err is None, err


def test_rne_bf16_against_the_oracle_rounding_and_torch_on_fp32():
    """The test-side rounding is itself pinned: equal to torch's cast on fp32-representable
    values (no double rounding there), and it rounds a fp64 value just above a bf16 midpoint
    up, which a detour through fp32 would turn into a tie rounded to even (down)."""
    g = torch.Generator().manual_seed(5)
    v = (torch.randn(20000, generator=g) * 3).to(torch.float32).to(f64)
    assert torch.equal(rne_bf16(v), v.to(torch.bfloat16).to(f64))
    x = torch.tensor([1.0 + 2.0 ** -8 + 2.0 ** -40], dtype=f64)       # midpoint of 1 and 1 + 2^-7, plus
    assert rne_bf16(x).item() == 1.0 + 2.0 ** -7
    assert x.to(torch.bfloat16).item() == 1.0                          # the fp32 detour ties to even
    np.testing.assert_array_equal(O.round_bf16(x.numpy()), rne_bf16(x).numpy())


# ---- the composition catches plausible mistakes in the oracle's layer --------------------------
# Each variant plants one mistake in a copy of the oracle's layer block (on the CPU only) and the
# comparison above must then fail.

def _block_norm_of_x(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = L.rnd(O.rms_norm(x, L.eps))                                   # wrong: normalises x, not h1
    act = L.rnd(O.silu(u2 @ L.wg.T) * (u2 @ L.wu.T))
    h2 = O.round_f32(h1 + act @ L.wd.T)
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2), "u3": L.rnd(O.rms_norm(h2, L.eps))}


def _block_silu_after_product(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = L.rnd(O.rms_norm(h1, L.eps))
    act = L.rnd(O.silu((u2 @ L.wg.T) * (u2 @ L.wu.T)))                # wrong: SiLU of the product
    h2 = O.round_f32(h1 + act @ L.wd.T)
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2), "u3": L.rnd(O.rms_norm(h2, L.eps))}


def _block_gate_up_swapped(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = L.rnd(O.rms_norm(h1, L.eps))
    act = L.rnd(O.silu(u2 @ L.wu.T) * (u2 @ L.wg.T))                  # wrong: SiLU on the up half
    h2 = O.round_f32(h1 + act @ L.wd.T)
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2), "u3": L.rnd(O.rms_norm(h2, L.eps))}


def _block_no_mlp_residual(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = L.rnd(O.rms_norm(h1, L.eps))
    act = L.rnd(O.silu(u2 @ L.wg.T) * (u2 @ L.wu.T))
    h2 = O.round_f32(act @ L.wd.T)                                    # wrong: residual dropped
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2), "u3": L.rnd(O.rms_norm(h2, L.eps))}


def _block_final_norm_of_h1(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = L.rnd(O.rms_norm(h1, L.eps))
    act = L.rnd(O.silu(u2 @ L.wg.T) * (u2 @ L.wu.T))
    h2 = O.round_f32(h1 + act @ L.wd.T)
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2),
            "u3": L.rnd(O.rms_norm(h1, L.eps))}                          # wrong: final norm of h1


def _block_mlp_residual_from_x(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = L.rnd(O.rms_norm(h1, L.eps))
    act = L.rnd(O.silu(u2 @ L.wg.T) * (u2 @ L.wu.T))
    h2 = O.round_f32(x + act @ L.wd.T)                                 # wrong: residual from x, not h1
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2), "u3": L.rnd(O.rms_norm(h2, L.eps))}


def _block_no_r5_rounding(L, x, o):
    h1 = O.round_f32(x + o @ L.wo.T)
    u2 = O.rms_norm(h1, L.eps)                                         # wrong: R5 skipped
    act = L.rnd(O.silu(u2 @ L.wg.T) * (u2 @ L.wu.T))
    h2 = O.round_f32(h1 + act @ L.wd.T)
    return {"h1": h1, "u2": u2, "act": act, "h2": h2, "hidden_out": L.rnd(h2), "u3": L.rnd(O.rms_norm(h2, L.eps))}


@pytest.mark.parametrize("mutant", [_block_norm_of_x, _block_silu_after_product, _block_gate_up_swapped,
                                    _block_no_mlp_residual, _block_final_norm_of_h1, _block_mlp_residual_from_x,
                                    _block_no_r5_rounding])
def test_planted_layer_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(OC, "layer_block", mutant)
    ref, got = _case(SMALL, 23, 90, 40, "causal")
    assert _agree(ref, got) is not None
