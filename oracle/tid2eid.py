"""Oracle: construction of the hash-routing table tid2eid.

Test infrastructure only (see the package docstring).

"How was DeepSeek V4's tid2eid derived?", section "Mathematical
formulation": m tokens with frequencies p_i (sorted descending), n experts,
k experts per token; x_{i,j} in {0,1} with sum_j x_{i,j} = k, and the load
sum_i p_i x_{i,j} should be close to k/n -- eq. (2) minimises
sum_j (sum_i p_i x_{i,j} - k/n)^2.

Greedy rule (same section and "Reference implementation"): take tokens by
decreasing frequency; give each the k experts whose current load is
smallest; add p_i / k to each of those loads (normalised loads f, so that
sum f = sum p).  Balance is reported as max_vio = max(f) * n - 1 and
min_vio = min(f) * n - 1.

Readings: equal frequencies are taken in ascending token id; equal loads go
to the lower expert id, and the k chosen ids are stored in ascending (load,
id) order, which is the order an argsort of the loads returns when it keeps
equal loads in index order.  The table is indexed by token id.

Pins: tests/test_oracle_tid2eid.py (brute-force optimum of eq. (2) on tiny
m, n; uniform p reaching objective 0; the extreme-case lower bound
max_vio >= p_1 n / k - 1 and its attainment; hand-worked fixtures in
tests/golden/tid2eid_small.json).
"""

import itertools

import numpy as np


def balance_violations(f, n):
    f = np.asarray(f, dtype=np.float64)
    return float(f.max() * n - 1.0), float(f.min() * n - 1.0)


def tid2eid_greedy(p, n, k):
    """Greedy least-loaded table. Returns (table [m,k] int32, f [n], max_vio, min_vio)."""
    p = np.asarray(p, dtype=np.float64)
    m = p.shape[0]
    token_order = np.lexsort((np.arange(m), -p))   # p descending, id ascending
    return tid2eid_greedy_order(p, n, k, token_order)


def tid2eid_greedy_order(p, n, k, token_order):
    """The greedy rule with tokens taken in `token_order` (a permutation of
    0..m-1) instead of by decreasing frequency -- the randomised variant of
    the "Reference implementation" section.  Same tie rules."""
    p = np.asarray(p, dtype=np.float64)
    m = p.shape[0]
    if not (0 < k <= n):
        raise ValueError("need 0 < k <= n")
    f = np.zeros(n, dtype=np.float64)
    table = np.zeros((m, k), dtype=np.int32)
    expert_ids = np.arange(n)
    for i in token_order:
        chosen = np.lexsort((expert_ids, f))[:k]   # load ascending, id ascending
        share = p[i] / k
        for j in chosen:
            f[j] += share
        table[i] = chosen
    max_vio, min_vio = balance_violations(f, n)
    return table, f, max_vio, min_vio


def tid2eid_objective(p, table, n, k):
    """Eq. (2): sum_j (sum_i p_i x_{i,j} - k/n)^2 for a table of expert ids."""
    p = np.asarray(p, dtype=np.float64)
    loads = np.zeros(n, dtype=np.float64)
    for i in range(table.shape[0]):
        for j in set(int(e) for e in table[i]):
            loads[j] += p[i]
    return float(np.sum((loads - k / n) ** 2))


def tid2eid_bruteforce(p, n, k):
    """Exact minimum of eq. (2) over every assignment of k distinct experts
    to each token (C(n,k)^m candidates: tiny m, n only)."""
    p = np.asarray(p, dtype=np.float64)
    m = p.shape[0]
    combos = list(itertools.combinations(range(n), k))
    best = np.inf
    best_table = None
    for choice in itertools.product(range(len(combos)), repeat=m):
        loads = np.zeros(n, dtype=np.float64)
        for i, c in enumerate(choice):
            for j in combos[c]:
                loads[j] += p[i]
        obj = float(np.sum((loads - k / n) ** 2))
        if obj < best:
            best = obj
            best_table = np.array([combos[c] for c in choice], dtype=np.int32)
    return best, best_table


def tid2eid_multistart(p, n, k, orders):
    """Run the greedy once per token order in `orders` [S, m] and keep the
    table with the smallest max_vio (the page's "run it multiple times and
    pick ... the lowest max_vio"); equal max_vio keeps the earlier start.
    Returns (table, f, max_vio, min_vio, best_start)."""
    best = None
    for s_idx, order in enumerate(orders):
        table, f, mx, mn = tid2eid_greedy_order(p, n, k, np.asarray(order))
        if best is None or mx < best[2]:
            best = (table, f, mx, mn, s_idx)
    return best
