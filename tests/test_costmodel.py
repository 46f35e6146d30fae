"""The Copy-as-Decode cost model (s(N), the Eq. (3) bounds, the minimum-span policy) against the
values the page prints: Table 11's s column from its AR and PP columns, Table 2's bnd_m8 and
bnd_N from Table 11's 7B curve, Table 17's m* (tests/golden/cad_kernel_table.json)."""
import json
import math
import os

import pytest

from spec_verify_cad_amd import costmodel as C

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cad_kernel_table.json")))


def _curve(model):
    t = GOLD["table11"][model]
    return C.s_curve(dict(zip(t["N"], t["ar"])), dict(zip(t["N"], t["pp"])))


def _half_unit(x: float) -> float:
    """Half a unit in the last printed digit of a table entry (integers above 100, else 0.1;
    the PP column prints one decimal throughout)."""
    return 0.5 if x >= 100 else 0.05


@pytest.mark.parametrize("model", ["qwen2.5-1.5b", "qwen2.5-7b"])
def test_s_column_of_the_kernel_table(model):
    """The page computes s from unrounded medians and prints AR, PP and s rounded, so s(N) from
    the printed AR and PP must agree with the printed s within the rounding of all three."""
    cur = _curve(model)
    t = GOLD["table11"][model]
    for n, ar, pp, s in zip(t["N"], t["ar"], t["pp"], t["s_printed"]):
        lo = (ar - _half_unit(ar)) / (pp + 0.05)
        hi = (ar + _half_unit(ar)) / (pp - 0.05)
        assert lo <= cur[n] <= hi
        assert lo - _half_unit(s) <= s <= hi + _half_unit(s), (n, lo, hi, s)


@pytest.mark.parametrize("row", GOLD["table2_7b"], ids=lambda r: r["corpus"])
def test_closed_form_bounds_of_table2(row):
    cur = _curve("qwen2.5-7b")
    assert abs(cur[8] - row["s_m8"]) < 0.01                    # 191 / 28.1 against the printed 6.79
    f = row["T_copy"] / row["T"]
    assert round(C.bound_uniform(f, row["s_m8"]), 2) == pytest.approx(row["bnd_m8"])
    digits = 1 if row["bnd_mean"] >= 10 or row["corpus"] == "ProbeEdit" else 2
    assert round(C.bound_uniform(f, C.interp_s(cur, row["mean_span"])), digits) == pytest.approx(row["bnd_mean"])


def test_minimum_span_policy_of_table17():
    t17 = GOLD["table17"]
    cur7 = _curve("qwen2.5-7b")
    assert C.m_star(cur7, t17["tau_ms"], t17["c_ms"]) == t17["qwen2.5-7b"]["strict"]
    assert C.m_safe(cur7) == t17["qwen2.5-7b"]["safe"]
    assert C.m_star(_curve("qwen2.5-1.5b"), t17["tau_ms"], t17["c_ms"]) == t17["qwen2.5-1.5b"]["strict"]
    # a fixed cost large against the span's AR time pushes m* up: c / (N tau) must fall below s - 1
    assert C.m_star(cur7, 1.0, 40.0) == 8                      # 6.80 > 1 + 40/8; 3.03 < 1 + 40/4


def test_interpolation_and_reductions():
    cur = _curve("qwen2.5-7b")
    for n in cur:
        assert C.interp_s(cur, n) == cur[n]
    assert C.interp_s(cur, 0.5) == cur[1] and C.interp_s(cur, 4096) == cur[512]
    mid = C.interp_s(cur, math.sqrt(16 * 32))                 # geometric midpoint: the mean of the ends
    assert mid == pytest.approx((cur[16] + cur[32]) / 2)
    # every span of one length: the exact bound is the uniform closed form
    spans = [24] * 50
    T = 1500
    assert C.bound_exact(spans, T, T - 1200, cur) == pytest.approx(C.bound_uniform(1200 / T, C.interp_s(cur, 24)))
    b = C.bounds(spans, T, cur)
    assert b["bnd_exact"] == pytest.approx(b["bnd_mean"]) and b["K"] == 50
    # Eq. (2) without splices or fixed costs is full regeneration
    assert C.cad_latency(20.0, 300, [], cur, 0, 1.0) == 6000.0
    assert C.cad_latency(20.0, 0, [8], cur, 1, 1.0) == pytest.approx(20.0 * 8 / cur[8] + 1.0)


def test_policy_edge_cases():
    flat = {1: 1.0, 2: 1.0, 4: 1.2, 8: 1.4}
    assert C.m_star(flat, 1.0, 0.0) == 4                        # s(2) = 1 is no gain
    assert C.m_safe(flat) is None                               # never above 1.5
    assert C.m_star(flat, 1.0, 100.0) is None                   # a fixed cost no span clears
    b = C.bounds([], 100, flat)                                 # no copies: full regeneration
    assert b["bnd_exact"] == 1.0 and b["bnd_mean"] == 1.0 and b["K"] == 0
