"""Pins of the oracle's n-gram lookup and acceptance scans.

n-gram lookup (PLD page, 'The n-gram match, precisely'): two independently written brute
forces agree exhaustively on tiny alphabets, plus hand-worked cases.  Acceptance (PLD
page, 'Verification in a single parallel pass'): the page's stated outcomes and an
exhaustive check against a prefix-comparison definition."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_ngram_hand_cases():
    ctx = [5, 1, 2, 3, 1, 2]
    d, l, m = O.ngram_lookup(ctx, 6, 2, 2, 3)          # suffix (1, 2) recurs at j = 1 only
    assert list(m) == [1, -1] and list(l) == [3, 0] and list(d[0]) == [3, 1, 2]
    ctx = [7, 7, 7, 7]                                  # overlapping matches, truncated at the end
    d, l, m = O.ngram_lookup(ctx, 4, 2, 3, 4)
    assert list(m) == [1, 0, -1] and list(l) == [1, 2, 0]
    assert list(d[0]) == [7, 0, 0, 0] and list(d[1]) == [7, 7, 0, 0]
    d, l, m = O.ngram_lookup([1, 2], 2, 2, 1, 3)        # too short: no candidate start
    assert list(m) == [-1] and list(l) == [0]
    d, l, m = O.ngram_lookup([1, 2, 3, 9, 9], 3, 1, 2, 2)   # only the first `length` tokens count
    assert list(m) == [-1, -1]


def test_ngram_two_brute_forces_agree_exhaustively():
    rng = np.random.default_rng(0)
    checked = 0
    for V in (1, 2, 3, 4):
        for length in range(0, 13):
            seqs = itertools.product(range(V), repeat=length) if V ** length <= 256 else \
                (tuple(rng.integers(0, V, size=length)) for _ in range(256))
            for seq in seqs:
                ctx = np.array(list(seq) + [V + 5] * 3, dtype=np.int64)   # junk beyond length
                for n in range(1, 5):
                    W, D = 1 + (length + n) % 4, 1 + (length * 3 + n) % 5
                    a = O.ngram_lookup(ctx, length, n, W, D)
                    b = O.ngram_lookup_bruteforce(ctx, length, n, W, D)
                    for x, y in zip(a, b):
                        np.testing.assert_array_equal(x, y)
                    checked += 1
    assert checked > 10000


def test_ngram_matches_really_match():
    rng = np.random.default_rng(1)
    for _ in range(300):
        L = int(rng.integers(1, 60))
        ctx = rng.integers(0, 3, size=L)
        n, W, D = int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 12))
        d, l, m = O.ngram_lookup(ctx, L, n, W, D)
        prev = L
        for w in range(W):
            if m[w] < 0:
                assert l[w] == 0 and all(m[w:] < 0)
                break
            j = int(m[w])
            assert j < prev and j + n <= L - 1
            assert list(ctx[j:j + n]) == list(ctx[L - n:])
            assert l[w] == min(D, L - j - n) and list(d[w, :l[w]]) == list(ctx[j + n:j + n + l[w]])
            prev = j


def test_accept_page_cases():
    cases = json.load(open(os.path.join(GOLD, "accept_scan_cases.json")))["cases"]
    for c in cases:
        a, em = O.accept_causal(c["draft"], len(c["draft"]), c["pred"])
        assert a == c["a"] and em == c["emitted"]


def test_accept_exhaustive_against_prefix_definition():
    # a is the largest i <= draft_len with draft[:i] == pred[:i]; emitted = draft[:a] + [pred[a]].
    for k in range(0, 5):
        for V in (1, 2, 3):
            for draft in itertools.product(range(V), repeat=k):
                for pred in itertools.product(range(V), repeat=k + 1):
                    for dl in range(0, k + 1):
                        a, em = O.accept_causal(draft, dl, pred)
                        want = max(i for i in range(dl + 1) if list(draft[:i]) == list(pred[:i]))
                        assert a == want
                        assert em == list(draft[:a]) + [pred[a]] and len(em) == a + 1


def test_accept_block_exhaustive_small():
    # Per-candidate runs against first_pred then the candidate's own predictions; the
    # longest wins, ties to the lowest candidate.
    rng = np.random.default_rng(2)
    for _ in range(3000):
        W, D = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        drafts = rng.integers(0, 2, size=(W, D))
        lens = rng.integers(0, D + 1, size=W)
        pred = rng.integers(0, 2, size=W * D)
        fp = int(rng.integers(0, 2))
        a, w, em, per = O.accept_block(drafts, lens, pred, fp, D)
        for c in range(W):
            seq_pred = [fp] + list(pred[c * D:(c + 1) * D - 1])
            want = max(i for i in range(lens[c] + 1) if list(drafts[c, :i]) == seq_pred[:i])
            assert per[c] == want
        assert a == max(per) and w == per.index(max(per))
        bonus = fp if a == 0 else int(pred[w * D + a - 1])
        assert em == list(drafts[w, :a]) + [bonus]


def test_commit_block_moves_winner_rows():
    c = O.Cache(1, 20, 2)
    c.length = 5
    c.K[0, :, 0] = np.arange(20)
    O.commit_block(c, w_star=2, a_star=3, D=4)
    assert c.length == 8
    np.testing.assert_array_equal(c.K[0, 5:8, 0], [13, 14, 15])


def test_pld_worked_example():
    g = json.load(open(os.path.join(GOLD, "pld_worked_example.json")))
    for c in g["cases"]:
        s = O.pld_speedup(c["f"], c["L"])
        assert round(s, c["digits"]) == c["speedup_printed"]
        if "passes_copied" in c:
            T, f, L = c["T"], c["f"], c["L"]
            assert f * T / L == c["passes_copied"] and round((1 - f) * T) == c["passes_new"]
            assert round(f * T / L + (1 - f) * T) == c["passes_total_approx"]
            assert abs(T / (f * T / L + (1 - f) * T) - s) < 1e-12


def test_ngram_longest_match_hand_case():
    # history ... 7 1 2 3 | 5 ... 1 2 3 ends: the 3-gram (1, 2, 3) recurs at j = 1; a 4-gram does not
    ctx = [7, 1, 2, 3, 5, 6, 4, 2, 3, 8, 1, 2, 3]
    d, l, m, n = O.ngram_lookup_longest(ctx, len(ctx), 4, 1, 1, 3)
    assert n == 3 and m[0] == 1 and list(d[0]) == [5, 6, 4] and l[0] == 3
    # with n_max = 2 the most recent 2-gram (2, 3) wins: j = 7, continuation (8, 1, 2)
    d, l, m, n = O.ngram_lookup_longest(ctx, len(ctx), 2, 1, 1, 3)
    assert n == 2 and m[0] == 7 and list(d[0]) == [8, 1, 2]
    d, l, m, n = O.ngram_lookup_longest([1, 2, 3, 4], 4, 3, 1, 2, 2)      # nothing recurs
    assert n == 0 and (m == -1).all() and (l == 0).all()


def test_ngram_longest_match_against_brute_force():
    """The length used is the largest with any earlier occurrence of the suffix (checked by a
    direct search), and the hits are those of the plain lookup at that length."""
    rng = np.random.default_rng(11)
    for _ in range(400):
        L = int(rng.integers(0, 40))
        ctx = rng.integers(0, 3, size=L)
        n_max, n_min = int(rng.integers(1, 6)), 1
        n_min = int(rng.integers(1, n_max + 1))
        d, l, m, n = O.ngram_lookup_longest(ctx, L, n_max, n_min, 2, 4)
        seq = [int(t) for t in ctx]

        def occurs(k):
            return L >= k + 1 and any(seq[j:j + k] == seq[L - k:] for j in range(0, L - k))

        want = next((k for k in range(n_max, n_min - 1, -1) if occurs(k)), 0)
        assert n == want
        if n:
            b = O.ngram_lookup_bruteforce(ctx, L, n, 2, 4)
            np.testing.assert_array_equal(d, b[0])
            np.testing.assert_array_equal(m, b[2])
        else:
            assert (m == -1).all()
