"""Oracle: auxiliary-loss-free bias update and expert-load statistics.

Test infrastructure only (see the package docstring).

"From One Giant FFN to 384 Tiny Experts", Ch.6 (the bias-update idea and
its pseudocode) and Ch.7.1 (V3's update speed 0.001): after a batch, every
routed expert i whose load is above the balanced level gets b_i -= gamma,
every expert below it gets b_i += gamma, and an expert exactly at the level
keeps its bias.  The bias only enters the top-k selection (Ch.6), so the
update changes no gate value.

Readings:
  * load_i is the number of (token, slot) pairs routed to expert i in the
    batch (the permutation's counts), and the balanced level is the mean
    load T*k/E.  The comparison is exact: load_i * E against T * k.
  * The bias is fp32 (the "gate-init" excerpt of "DeepSeek-V3.2-Exp -
    Routing weights" creates it as float32) and gamma is an fp32 value, so
    b -/+ gamma is one fp32 operation.
  * Load statistics, as the per-layer load-variance table of the MaxText
    pull request "Load balancing changes for Deepseek v4" reports them: the
    population variance of the per-expert counts; and, as the tid2eid page
    evaluates balance, max_vio = max(f) * n - 1 and min_vio = min(f) * n - 1
    with f_i = load_i / (T * k).

Pins: tests/test_oracle_balance.py (hand-worked batches; the balanced and
gamma = 0 fixed points; variance against the textbook two-pass formula in
exact rational arithmetic; monotone convergence of a two-expert toy system).
"""

from fractions import Fraction

import numpy as np


def load_stats(counts, T, k):
    """(mean, variance, max_vio, min_vio) of the expert loads `counts` [E]
    of a batch of T tokens with k experts each."""
    counts = [int(c) for c in counts]
    E = len(counts)
    total = T * k
    mean = Fraction(total, E)
    var = sum((Fraction(c) - mean) ** 2 for c in counts) / E
    max_vio = Fraction(max(counts) * E, total) - 1 if total else Fraction(0)
    min_vio = Fraction(min(counts) * E, total) - 1 if total else Fraction(0)
    return float(mean), float(var), float(max_vio), float(min_vio)


def bias_update(bias, counts, T, k, gamma):
    """New fp32 bias after one sign step of size gamma (fp32)."""
    bias = np.asarray(bias, dtype=np.float32)
    g = np.float32(gamma)
    E = bias.shape[0]
    out = bias.copy()
    for i in range(E):
        lhs, rhs = int(counts[i]) * E, T * k
        if lhs > rhs:
            out[i] = np.float32(bias[i] - g)       # overloaded: harder to select
        elif lhs < rhs:
            out[i] = np.float32(bias[i] + g)       # underloaded: easier to select
    return out
