"""Algorithmic bytes and flops of the span forward and its kernels, and MI355X peaks.

"Algorithmic" means what the method must move or compute at minimum: every weight read
once, the embedding rows of the new tokens, the visible K/V read once per KV head, the new
K/V rows written, the outputs written; flops are 2 per multiply-add of the projections and
LM head plus the attention score and value products over the visible keys.  Workspace
traffic of an implementation is not counted.
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3


def weight_bytes(s) -> int:
    return (s.layer_params() + s.lm_params()) * s.elt_bytes


def kv_row_bytes(s) -> int:
    """Bytes of one cached position (K and V, all KV heads)."""
    return 2 * s.n_kv_heads * s.head_dim * s.elt_bytes


def visible_keys_causal(L: int, N: int) -> float:
    """Sum over the N span rows of the keys each one attends to (cache L, causal span)."""
    return N * L + N * (N + 1) / 2


def forward_bytes(s, B: int, N: int, L: int, hidden_out: bool = False) -> float:
    """One causal span forward of N rows per sequence over caches of length L."""
    b = weight_bytes(s)
    b += B * N * s.hidden * s.elt_bytes                 # embedding rows
    b += B * (L + N) * kv_row_bytes(s)                  # K/V read once per KV head (incl. the new rows)
    b += B * N * kv_row_bytes(s)                        # K/V rows appended
    b += B * N * 4                                      # argmax out
    b += B * N * 4 * 2                                  # tokens in, nothing else
    if hidden_out:
        b += B * N * s.hidden * s.elt_bytes
    return float(b)


def forward_flops(s, B: int, N: int, L: int, visible: float | None = None) -> float:
    """2 * rows * params for the projections and LM head plus 4 * d * Hq per visible key."""
    vis = visible_keys_causal(L, N) if visible is None else visible
    return 2.0 * B * N * (s.layer_params() + s.lm_params()) + 4.0 * B * vis * s.n_q_heads * s.head_dim


def lm_head_bytes(s, M: int) -> float:
    """LM head + argmax: the vocab x hidden weight once, M normed rows in, M ids out."""
    return float(s.vocab * s.hidden * s.elt_bytes + M * s.hidden * s.elt_bytes + M * 4)


def lm_head_flops(s, M: int) -> float:
    return 2.0 * M * s.hidden * s.vocab


def floor_us(nbytes: float, flops: float) -> tuple:
    """(time floor in us, bound) from HBM and bf16 MFMA peaks."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
    return (t_hbm, "hbm") if t_hbm >= t_mfma else (t_mfma, "mfma")


def pld_round_bytes(s, B: int, k: int, L: int, ctx_len: int) -> float:
    """One batched PLD round: the n-gram scan of every history (int32), a verify forward of k + 1
    rows per sequence over caches of length L, and the accept scan's few bytes per sequence."""
    return forward_bytes(s, B, k + 1, L) + B * ctx_len * 4 + B * (k + 1) * 4 * 4


def pld_round_flops(s, B: int, k: int, L: int) -> float:
    return forward_flops(s, B, k + 1, L)


def stack_forward_bytes(s, n_layers: int, B: int, N: int, L: int, last_only: bool = False) -> float:
    """One causal span forward through a stack: every layer's weights and the LM head once, the
    embedding rows, and per layer the visible K/V read once plus the new rows written."""
    b = (n_layers * s.layer_params() + s.lm_params()) * s.elt_bytes
    b += B * N * s.hidden * s.elt_bytes
    b += n_layers * B * ((L + N) + N) * kv_row_bytes(s)
    b += B * (1 if last_only else N) * 4 + B * N * 4
    return float(b)


def stack_forward_flops(s, n_layers: int, B: int, N: int, L: int, last_only: bool = False) -> float:
    lm_rows = B * (1 if last_only else N)
    return (2.0 * B * N * n_layers * s.layer_params() + 2.0 * lm_rows * s.lm_params()
            + 4.0 * n_layers * B * visible_keys_causal(L, N) * s.n_q_heads * s.head_dim)


def med_iqr(samples) -> dict:
    """Median and interquartile range of timing samples (linear-interpolated quartiles), with
    the sample count."""
    xs = sorted(float(x) for x in samples)
    n = len(xs)

    def q(p):
        t = p * (n - 1)
        i = int(t)
        return xs[i] if i + 1 >= n else xs[i] + (xs[i + 1] - xs[i]) * (t - i)

    return {"median": round(q(0.5), 2), "q1": round(q(0.25), 2), "q3": round(q(0.75), 2),
            "iqr": round(q(0.75) - q(0.25), 2), "n": n}
