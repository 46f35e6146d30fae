"""Pins of the oracle's stochastic verification (PLD page: with the rejection-sampling
correction, speculative verification keeps the target's sampling distribution).

* The Philox4x32-10 stream is uniform bit by bit and byte by byte, and the uniforms built from
  it are fp32-exact and never 0 or 1.
* Distribution preservation: over many seeds, the token a one-draft verification emits first
  (the kept draft or the replacement draw) is distributed as softmax(logits / T), whichever
  token was drafted; so is a plain draw; and a replacement never repeats the draft.
* Limits: at a small temperature the draws collapse to the argmax, a draft equal to the argmax
  is kept and any other draft is replaced by the argmax."""
import math

import numpy as np
import pytest

import oracle as O

CHI2_5DOF_1E4 = 25.74      # chi-square quantile, 5 degrees of freedom, upper tail 1e-4


def test_philox_stream_is_uniform():
    n = 1 << 14
    ctr = np.stack([np.arange(n), np.zeros(n), np.full(n, 3), np.zeros(n)], axis=-1).astype(np.uint64)
    w = O.philox4x32_10(ctr, (12345, 678)).reshape(-1)
    bits = ((w[:, None] >> np.arange(32, dtype=np.uint32)) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 4 * 0.5 / math.sqrt(w.size))
    hist = np.bincount((w >> 24).astype(np.int64), minlength=256)
    exp = w.size / 256
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)                # mean 255, sd sqrt(510)
    # another key, another stream; neighbouring counters share no words
    w2 = O.philox4x32_10(ctr, (12346, 678)).reshape(-1)
    assert np.mean(w == w2) < 1e-3
    assert len(np.unique(w)) > 0.999 * w.size


def test_uniforms_are_exact_fp32_and_open():
    bits = np.array([0, 1, 511, 512, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = O.uniform_from_bits(bits)
    assert u[0] == 2.0 ** -24 and u[4] == 1 - 2.0 ** -24
    assert u[2] == u[0] and u[3] == 3 * 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)
    assert np.all((u > 0) & (u < 1))


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("d", [0, 2, 5])
def test_first_emitted_token_has_the_target_distribution(d):
    logits = np.array([[1.2, -0.3, 0.8, 2.0, -1.0, 0.1], [0.0, 0.5, -0.5, 1.0, 0.2, -0.2]])
    T = 0.8
    p = _softmax(logits[0] / T)
    n = 6000
    first = np.zeros(6, dtype=np.int64)
    plain = np.zeros(6, dtype=np.int64)
    for seed in range(n):
        pred, y, z, pd, u = O.sampled_predictions(logits, [7, d], 1, T, seed, 0, 100)
        assert z[0] != d and pred[0] in (d, z[0])
        assert pd[0] == pytest.approx(p[d])
        first[pred[0]] += 1
        plain[y[0]] += 1
    for counts in (first, plain):
        chi2 = float(np.sum((counts - n * p) ** 2 / (n * p)))
        assert chi2 < CHI2_5DOF_1E4, (counts, n * p)


def test_small_temperature_limits():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((3, 50))
    T = 1e-3
    top = np.argmax(logits, axis=1)
    for seed in range(20):
        toks = [9, int(top[0]), (int(top[1]) + 1) % 50]
        pred, y, z, pd, u = O.sampled_predictions(logits, toks, 2, T, seed, 1, 7)
        assert list(y) == list(top)
        assert pred[0] == top[0]                       # draft = argmax: kept
        assert pred[1] == top[1] and z[1] == top[1]    # another draft: replaced by the argmax
        assert pred[2] == top[2]                       # the bonus row: a plain draw


def test_draws_are_keyed_by_sequence_position_and_seed():
    logits = np.zeros((2, 64))                         # uniform target: the draw is the noise argmax
    a = O.sampled_predictions(logits, [1, 2], 0, 1.0, 11, 0, 40)[1]
    b = O.sampled_predictions(logits[::-1], [5, 6], 0, 1.0, 11, 0, 40)[1]
    assert list(a) == list(b)                          # same (seed, b, positions), same draws
    c = O.sampled_predictions(logits, [1, 2], 0, 1.0, 11, 0, 41)[1]
    assert c[0] == a[1]                                # position 41 is row 1 above
    draws = [O.sampled_predictions(logits[:1], [1], 0, 1.0, s, 0, 40)[1][0] for s in range(200)]
    assert len(set(draws)) > 40                        # seeds give different draws
