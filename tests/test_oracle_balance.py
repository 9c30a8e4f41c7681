"""Pins of the oracle's bias update and load statistics ("From One Giant FFN
to 384 Tiny Experts", Ch.6 and 7.1; the load-variance table of the MaxText
pull request "Load balancing changes for Deepseek v4")."""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _f32_exact(v):
    return Fraction(float(np.float32(v)))


def test_hand_worked_batch():
    # T = 4 tokens, k = 3 -> 12 pairs over E = 3 experts: balanced level 4
    counts = [5, 3, 4]
    bias = np.array([0.1, -0.2, 0.0], dtype=np.float32)
    new = oracle.bias_update(bias, counts, 4, 3, 0.001)
    assert new.dtype == np.float32
    g = _f32_exact(0.001)
    # one correctly rounded fp32 step, checked in exact rational arithmetic
    for i, sign in ((0, -1), (1, +1)):
        exact = _f32_exact(bias[i]) + sign * g
        got = Fraction(float(new[i]))
        ulp = Fraction(float(np.spacing(np.float32(abs(float(exact))))))
        assert abs(got - exact) <= ulp / 2
    assert new[2] == bias[2]                     # exactly at the level: unchanged
    mean, var, mx, mn = oracle.load_stats(counts, 4, 3)
    assert mean == 4.0 and var == pytest.approx(2.0 / 3.0, rel=1e-15)
    assert mx == pytest.approx(0.25) and mn == pytest.approx(-0.25)


def test_fixed_points():
    bias = np.linspace(-0.05, 0.05, 16).astype(np.float32)
    same = oracle.bias_update(bias, [8] * 16, 16, 8, 0.001)      # perfectly balanced
    np.testing.assert_array_equal(same, bias)
    rng = np.random.default_rng(0)
    counts = rng.multinomial(128, np.ones(16) / 16)
    np.testing.assert_array_equal(oracle.bias_update(bias, counts, 16, 8, 0.0), bias)


def test_statistics_match_textbook_formulas():
    rng = np.random.default_rng(3)
    for E, T, k in ((256, 4096, 8), (384, 8192, 8), (7, 5, 3)):
        counts = rng.multinomial(T * k, rng.dirichlet(np.ones(E)))
        mean, var, mx, mn = oracle.load_stats(counts, T, k)
        assert mean == pytest.approx(T * k / E, rel=1e-15)
        assert var == pytest.approx(np.var(counts.astype(np.float64)), rel=1e-12)
        f = counts / (T * k)
        emx, emn = oracle.balance_violations(f, E)
        assert mx == pytest.approx(emx, rel=1e-12, abs=1e-15)
        assert mn == pytest.approx(emn, rel=1e-12, abs=1e-15)


def test_control_loop_balances_a_toy_router():
    """Two experts, k = 1: token t picks the expert with the larger s + b.
    Repeated sign steps must drive the loads towards T/2 (a wrong sign would
    push every token onto one expert)."""
    rng = np.random.default_rng(5)
    T = 400
    s = rng.normal(size=(T, 2)) + np.array([0.3, 0.0])   # expert 0 favoured
    bias = np.zeros(2, dtype=np.float32)
    first = None
    for _ in range(400):
        pick = np.argmax(s + bias, axis=1)
        counts = np.bincount(pick, minlength=2)
        first = counts if first is None else first
        bias = oracle.bias_update(bias, counts, T, 1, 0.01)
    assert abs(first[0] - T / 2) > 40
    assert abs(counts[0] - T / 2) <= 12
