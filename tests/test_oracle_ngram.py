"""Pins of the oracle's 2-gram hash gate ("How was DeepSeek V4's tid2eid
derived?", section "An extreme case")."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_small.json")


def _is_prime_mr(q):
    """Deterministic Miller-Rabin for q < 3.3e24 (bases of the first 12 primes)."""
    if q < 2:
        return False
    small = (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37)
    for b in small:
        if q % b == 0:
            return q == b
    d, r = q - 1, 0
    while d % 2 == 0:
        d //= 2
        r += 1
    for a in small:
        x = pow(a, d, q)
        if x in (1, q - 1):
            continue
        for _ in range(r - 1):
            x = pow(x, 2, q)
            if x == q - 1:
                break
        else:
            return False
    return True


def test_hand_worked_pairs():
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        w, idx = oracle.ngram_hash_gate([c["prev"]], [c["tok"]], g["vocab_size"], g["n_experts"],
                                        g["k"])
        assert idx[0].tolist() == c["experts"], c["work"]
        np.testing.assert_allclose(w[0], 1.0 / g["k"])


@pytest.mark.parametrize("m,k", [(10, 3), (32768, 4), (129280, 16), (1, 2), (2, 5)])
def test_primes_are_the_smallest_above_m(m, k):
    q = oracle.smallest_primes_above(m, k)
    assert len(q) == k and q[0] > m and all(b > a for a, b in zip(q, q[1:]))
    assert all(_is_prime_mr(v) for v in q)
    # no prime is skipped between m and the last one
    for v in range(m + 1, q[-1]):
        assert _is_prime_mr(v) == (v in q)


def test_zero_previous_token_gives_b_mod_n():
    rng = np.random.default_rng(0)
    b = rng.integers(0, 1000, size=50)
    _, idx = oracle.ngram_hash_gate(np.zeros(50, dtype=np.int64), b, 1000, 48, 6)
    np.testing.assert_array_equal(idx, np.repeat((b % 48)[:, None], 6, axis=1))


def test_route_scale_and_sequence_start():
    w, idx = oracle.ngram_hash_gate([-1, 5], [4, 4], 100, 7, 2, route_scale=2.5)
    np.testing.assert_allclose(w, 1.25)
    q = oracle.smallest_primes_above(100, 2)
    assert idx[0].tolist() == [(100 * q[0] + 4) % 7, (100 * q[1] + 4) % 7]


def test_random_pairs_are_nearly_balanced():
    """The page's claim for n-gram inputs: almost perfectly balanced loads."""
    rng = np.random.default_rng(1)
    m, n, k, T = 32768, 64, 4, 20000
    a = rng.integers(0, m, size=T)
    b = rng.integers(0, m, size=T)
    _, idx = oracle.ngram_hash_gate(a, b, m, n, k)
    load = np.bincount(idx.ravel(), minlength=n)
    mean = T * k / n
    assert np.abs(load - mean).max() < 6 * np.sqrt(mean)
