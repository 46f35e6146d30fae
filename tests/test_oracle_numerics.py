"""Pins of the oracle's number formats and element-wise building blocks against
library routines, closed forms and hand-worked cases."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def torch_bf16(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_on_fp32_values():
    # For inputs that are exact fp32 values a single RNE step to bf16 is what torch's cast does.
    rng = np.random.default_rng(0)
    for scale in (1e-30, 1e-5, 0.02, 1.0, 3e3, 1e30):
        x = (rng.standard_normal(200000) * scale).astype(np.float32)
        np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), torch_bf16(x))


def test_round_bf16_hand_cases():
    u = 2.0 ** -7                                   # bf16 spacing on [1, 2)
    cases = [
        (1.0 + u / 2, 1.0),                         # tie, kept LSB even -> down
        (1.0 + 3 * u / 2, 1.0 + 2 * u),             # tie, kept LSB odd -> up
        (1.0 + u / 2 + 2.0 ** -40, 1.0 + u),        # just above a tie; fp32 first would tie-round down
        (1.0 + u / 2 - 2.0 ** -40, 1.0),
        (2.0 - u / 2, 2.0),                         # carry into the exponent
        (-(1.0 + 3 * u / 2), -(1.0 + 2 * u)),       # sign symmetry
        (0.0, 0.0),
    ]
    for x, want in cases:
        assert O.round_bf16(np.array([x]))[0] == want, (x, want)


def test_round_f32_matches_numpy_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000)
    np.testing.assert_array_equal(O.round_f32(x), x.astype(np.float32).astype(np.float64))


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96)) * 3
    ref = F.rms_norm(torch.from_numpy(x), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, 1e-6), ref, rtol=1e-13, atol=0)
    # with eps -> 0 the mean square of the output is 1
    np.testing.assert_allclose(np.mean(O.rms_norm(x, 0.0) ** 2, axis=-1), 1.0, rtol=1e-13)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_rope_identity_at_position_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 3, 64))
    np.testing.assert_array_equal(O.apply_rope(x, [0], 10000.0), x)


def test_rope_equals_complex_rotation():
    # Half-split RoPE is multiplication of (x_i + i x_{i+d/2}) by exp(i * p * base^(-2i/d)).
    rng = np.random.default_rng(4)
    d, base = 128, 10000.0
    x = rng.standard_normal((5, 2, d))
    pos = np.array([0, 1, 7, 2047, 33119])
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    theta = pos[:, None] * np.power(base, -np.arange(0, d, 2) / d)[None, :]
    rz = z * np.exp(1j * theta)[:, None, :]
    want = np.concatenate([rz.real, rz.imag], axis=-1)
    np.testing.assert_allclose(O.apply_rope(x, pos, base), want, rtol=0, atol=1e-12)


def test_rope_preserves_norm_and_is_relative():
    rng = np.random.default_rng(5)
    d = 128
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for m, n in [(3, 1), (100, 40), (2048, 2000)]:
        rq, rk = O.apply_rope(q, [m], 1e4), O.apply_rope(k, [n], 1e4)
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
        s0 = float(np.sum(rq * rk))
        for shift in (1, 17, 512):
            s1 = float(np.sum(O.apply_rope(q, [m + shift], 1e4) * O.apply_rope(k, [n + shift], 1e4)))
            assert abs(s1 - s0) < 1e-9


def test_softmax_rows_sum_to_one_and_mask():
    s = np.array([[0.0, 1.0, -np.inf, 2.0], [5.0, -np.inf, -np.inf, -np.inf]])
    p = O.softmax_checked(s)
    assert p[0, 2] == 0 and p[1, 0] == 1.0
    e = np.exp([0.0, 1.0, 2.0])
    np.testing.assert_allclose(p[0, [0, 1, 3]], e / e.sum(), rtol=1e-15)


def test_decode_bf16_bits():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4049, 0x3C00], dtype=np.uint16)
    np.testing.assert_array_equal(O.decode_bf16_bits(bits), [1.0, -1.0, 0.0, 3.140625, 2.0 ** -7])


def test_argmax_lowest_and_gap():
    lg = np.array([[1.0, 3.0, 3.0, 2.0], [0.5, 0.25, 0.5, 0.0]])
    np.testing.assert_array_equal(O.argmax_lowest(lg), [1, 0])
    np.testing.assert_array_equal(O.top2_gap(lg), [0.0, 0.0])
    assert O.top2_gap(np.array([[1.0, 4.0, 2.5]]))[0] == 1.5
