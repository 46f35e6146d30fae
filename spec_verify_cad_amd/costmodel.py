"""The Copy-as-Decode cost model evaluated on measured span-forward times (host arithmetic).

* s(N): the per-span speedup of one parallel forward of N tokens over N autoregressive steps,
  AR(N) / PP(N) (Copy-as-Decode §4.1 and Table 11).
* s at an unmeasured N: linear in log2 N between the measured neighbours (the log-linear
  interpolation the page uses for its exact bound, Table 2), held constant beyond the ends.
* Eq. (3): Speedup <= T / (T_gen + sum_k N_k / s(N_k)); the two closed forms that bracket it
  put every span at one length: 1 / ((1 - f) + f / s(N)) with f = T_copy / T, at the mean
  span length (aspirational) or at the minimum viable length m (conservative).
* Appendix J: a splice of N tokens pays when N*tau > N*tau/s(N) + c, so the minimum span is
  m* = min{N : s(N) > 1 + c / (N tau)}; the "safe" threshold is the first N with s(N) > 1.5.
  Spans start at N = 2 (a one-token "splice" is a decode step).
"""
from __future__ import annotations

import math


def s_curve(ar_ms: dict, pp_ms: dict) -> dict:
    """{N: AR(N) / PP(N)} from two {N: ms} tables."""
    return {int(n): ar_ms[n] / pp_ms[n] for n in sorted(ar_ms) if n in pp_ms}


def interp_s(curve: dict, n: float) -> float:
    """s at span length n: linear in log2 n between the measured neighbours, constant outside."""
    ns = sorted(curve)
    if n <= ns[0]:
        return curve[ns[0]]
    if n >= ns[-1]:
        return curve[ns[-1]]
    for lo, hi in zip(ns, ns[1:]):
        if lo <= n <= hi:
            t = (math.log2(n) - math.log2(lo)) / (math.log2(hi) - math.log2(lo))
            return curve[lo] + t * (curve[hi] - curve[lo])
    raise AssertionError("unreachable")


def bound_uniform(f: float, s: float) -> float:
    """1 / ((1 - f) + f / s): every copied token spliced at speedup s."""
    return 1.0 / ((1.0 - f) + f / s)


def bound_exact(spans, T: int, T_gen: int, curve: dict) -> float:
    """Eq. (3) over an explicit list of copy-span lengths."""
    return T / (T_gen + sum(n / interp_s(curve, n) for n in spans))


def bounds(spans, T: int, curve: dict, m: int = 8) -> dict:
    """The three bounds of a program: exact over its span histogram, at the mean span length,
    and at the minimum viable length m."""
    T_copy = sum(spans)
    T_gen = T - T_copy
    f = T_copy / T
    nbar = T_copy / len(spans) if spans else 0.0
    return {"T": T, "T_copy": T_copy, "T_gen": T_gen, "f": f, "K": len(spans), "mean_span": nbar,
            "s_m": interp_s(curve, m), "bnd_m": bound_uniform(f, interp_s(curve, m)),
            "bnd_mean": bound_uniform(f, interp_s(curve, nbar)) if spans else 1.0,
            "bnd_exact": bound_exact(spans, T, T_gen, curve)}


def m_star(curve: dict, tau_ms: float, c_ms: float, n_min: int = 2):
    """Smallest measured N >= n_min with s(N) > 1 + c / (N tau), or None."""
    for n in sorted(curve):
        if n >= n_min and curve[n] > 1.0 + c_ms / (n * tau_ms):
            return n
    return None


def m_safe(curve: dict, threshold: float = 1.5, n_min: int = 2):
    """Smallest measured N >= n_min with s(N) > threshold, or None."""
    for n in sorted(curve):
        if n >= n_min and curve[n] > threshold:
            return n
    return None


def cad_latency(tau_ms: float, T_gen: int, spans, curve: dict, K: int, c_op_ms: float) -> float:
    """Eq. (2): tau*T_gen + tau * sum N_k/s(N_k) + K * (per-op fixed cost)."""
    return tau_ms * T_gen + tau_ms * sum(n / interp_s(curve, n) for n in spans) + K * c_op_ms
