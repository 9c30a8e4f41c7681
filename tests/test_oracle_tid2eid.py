"""Pins of the oracle's greedy tid2eid construction (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "tid2eid_small.json")))["cases"])
def test_hand_worked_cases(case):
    table, f, _, _ = oracle.tid2eid_greedy(np.array(case["p"]), case["n"], case["k"])
    assert table.tolist() == case["table"]
    np.testing.assert_allclose(f, case["load"], rtol=0, atol=1e-15)
    if "objective" in case:
        assert oracle.tid2eid_objective(np.array(case["p"]), table, case["n"], case["k"]) == \
            pytest.approx(case["objective"], abs=1e-15)


@pytest.mark.parametrize("m,n,k,seed", [(5, 4, 2, 0), (6, 3, 1, 1), (6, 4, 2, 2), (4, 4, 3, 3)])
def test_greedy_vs_bruteforce_optimum(m, n, k, seed):
    """Eq. (2) optimum over all C(n,k)^m assignments bounds the greedy result;
    the gap stays small on these instances."""
    p = np.sort(np.random.default_rng(seed).dirichlet(np.ones(m)))[::-1]
    table, _, _, _ = oracle.tid2eid_greedy(p, n, k)
    greedy = oracle.tid2eid_objective(p, table, n, k)
    best, best_table = oracle.tid2eid_bruteforce(p, n, k)
    assert best <= greedy + 1e-15
    assert oracle.tid2eid_objective(p, best_table, n, k) == pytest.approx(best, abs=1e-15)
    assert greedy - best <= 0.05


def test_bruteforce_finds_known_optimum():
    # p = [.4,.3,.2,.1], n = 2, k = 1: {.4,.1} / {.3,.2} splits evenly -> 0
    best, table = oracle.tid2eid_bruteforce(np.array([0.4, 0.3, 0.2, 0.1]), 2, 1)
    assert best == pytest.approx(0.0, abs=1e-15)
    # two tokens of 0.5 on 2 experts with k = 1: one each -> 0; never both on one
    best, table = oracle.tid2eid_bruteforce(np.array([0.5, 0.5]), 2, 1)
    assert best == pytest.approx(0.0, abs=1e-15) and table[0, 0] != table[1, 0]


@pytest.mark.parametrize("m,n,k", [(64, 16, 4), (48, 8, 2), (30, 6, 6)])
def test_uniform_frequencies_balance_exactly(m, n, k):
    """m*k divisible by n and equal p: the greedy fills experts round-robin and
    every load is exactly 1/n, so eq. (2) is 0 and max_vio = min_vio = 0."""
    p = np.full(m, 1.0 / m)
    table, f, mx, mn = oracle.tid2eid_greedy(p, n, k)
    np.testing.assert_allclose(f, 1.0 / n, rtol=1e-12)
    assert abs(mx) < 1e-12 and abs(mn) < 1e-12
    assert oracle.tid2eid_objective(p, table, n, k) < 1e-24
    assert all(len(set(r)) == k for r in table.tolist())


def test_extreme_token_lower_bound_is_attained():
    """A token with p_1 > k/n puts p_1 on each of its k experts ("An extreme
    case"): no table has max_vio below p_1*n/k - 1, and on the Zipf(1.1)
    vocabulary of 32768 ids with n = 64, k = 4 the greedy attains it."""
    m, n, k = 32768, 64, 4
    p = np.arange(1, m + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    assert p[0] > k / n
    table, f, mx, mn = oracle.tid2eid_greedy(p, n, k)
    assert mx == pytest.approx(p[0] * n / k - 1.0, rel=1e-12)
    assert 1.2698 < mx < 1.2699
    assert table[0].tolist() == [0, 1, 2, 3]
    assert f.sum() == pytest.approx(1.0, rel=1e-12)
    assert all(len(set(r)) == k for r in table[:2000].tolist())
    # eq. (2) lower bound from the extreme token alone
    assert oracle.tid2eid_objective(p, table, n, k) >= k * (p[0] - k / n) ** 2


def test_extreme_bound_holds_for_bruteforce_optimum():
    p = np.array([0.55, 0.2, 0.15, 0.1])
    n, k = 4, 2                                    # k/n = .5 < p_1
    best, _ = oracle.tid2eid_bruteforce(p, n, k)
    assert best >= k * (p[0] - k / n) ** 2 - 1e-15


def test_rows_distinct_and_mass_conserved():
    rng = np.random.default_rng(4)
    p = rng.random(500)
    p /= p.sum()
    table, f, mx, mn = oracle.tid2eid_greedy(p, 32, 5)
    assert all(len(set(r)) == 5 for r in table.tolist())
    assert f.sum() == pytest.approx(1.0, rel=1e-12)
    assert mx == pytest.approx(f.max() * 32 - 1) and mn == pytest.approx(f.min() * 32 - 1)


# --- randomised multi-start variant ("Reference implementation": process the
# tokens in a random order, run several times, keep the lowest max_vio) ---

def test_frequency_order_reproduces_the_greedy():
    rng = np.random.default_rng(11)
    p = np.sort(rng.dirichlet(np.ones(300)))[::-1]
    t1, f1, mx1, mn1 = oracle.tid2eid_greedy(p, 16, 4)
    order = np.lexsort((np.arange(300), -p))
    t2, f2, mx2, mn2 = oracle.tid2eid_greedy_order(p, 16, 4, order)
    np.testing.assert_array_equal(t1, t2)
    assert (mx1, mn1) == (mx2, mn2)


def test_multistart_hand_worked():
    # m = 3, n = 2, k = 1, p = (.5, .3, .2)
    # order (0,1,2): e0 <- .5, e1 <- .3, e1 <- .2 -> loads (.5, .5), max_vio 0
    # order (2,1,0): e0 <- .2, e1 <- .3, e0 <- .5 -> loads (.7, .3), max_vio .4
    p = np.array([0.5, 0.3, 0.2])
    table, f, mx, mn, best = oracle.tid2eid_multistart(p, 2, 1, [[2, 1, 0], [0, 1, 2]])
    assert best == 1
    assert table[:, 0].tolist() == [0, 1, 1]
    assert mx == pytest.approx(0.0, abs=1e-15) and mn == pytest.approx(0.0, abs=1e-15)
    t_bad, _, mx_bad, _ = oracle.tid2eid_greedy_order(p, 2, 1, np.array([2, 1, 0]))
    assert t_bad[:, 0].tolist() == [0, 1, 0] and mx_bad == pytest.approx(0.4)


def test_multistart_keeps_the_earliest_of_equal_starts():
    p = np.array([0.4, 0.3, 0.2, 0.1])
    _, _, _, _, best = oracle.tid2eid_multistart(p, 2, 1, [[0, 1, 2, 3]] * 3)
    assert best == 0


def test_multistart_is_never_worse_than_any_start():
    rng = np.random.default_rng(2)
    p = rng.dirichlet(np.ones(200) * 0.3)
    orders = [rng.permutation(200) for _ in range(6)]
    _, f, mx, _, best = oracle.tid2eid_multistart(p, 8, 2, orders)
    for o in orders:
        assert mx <= oracle.tid2eid_greedy_order(p, 8, 2, o)[2]
    assert f.sum() == pytest.approx(p.sum())
